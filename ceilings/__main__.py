"""python -m ceilings: build libpipeceil.so (benchmark support)."""
from ceilings import build

print(build(verbose=True))
