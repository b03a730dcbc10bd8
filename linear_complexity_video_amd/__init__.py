"""MI355X-native forward core of LinGen's MATE block (RMS, bidirectional
Mamba2 scan with review tokens, TESA), as hand-written HIP for gfx950 behind a
C ABI (``include/mate.h``). The Python side only marshals arguments."""
