"""CPU oracle of the rasteriser: test infrastructure only (tests, smoke check, CPU baseline)."""
