// Decode kernels with 8 waves per workgroup (see decode_impl.inc).
#define SPEAR_WAVES 8
#define SPEAR_DECODE_NS w8
#include "decode_impl.inc"
