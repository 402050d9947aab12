"""MI355X (gfx950) hybrid sparse attention forward: HCA / CSA / SWA."""
