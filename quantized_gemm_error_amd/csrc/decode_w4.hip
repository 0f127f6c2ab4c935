// Decode kernels with 4 waves per workgroup (see decode_impl.inc).
#define SPEAR_WAVES 4
#define SPEAR_DECODE_NS w4
#include "decode_impl.inc"
