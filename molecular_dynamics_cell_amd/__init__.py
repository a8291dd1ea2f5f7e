"""REANN-style message-passing interatomic potential: energy/force hot path on MI355X (gfx950)."""
