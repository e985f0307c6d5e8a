"""Reader for the small key/value fixtures in this folder (comment lines start with #)."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            nums = []
            for v in vals:
                try:
                    nums.append(int(v))
                except ValueError:
                    nums.append(float(v))
            out[key] = nums[0] if len(nums) == 1 else nums
    return out
