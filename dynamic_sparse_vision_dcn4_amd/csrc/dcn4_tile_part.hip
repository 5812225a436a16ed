// dcn4_tile_part.hip -- the tiled forward kernels of one (dtype, sampling
// mode) pair, DCN4_TILE_PART_DT and DCN4_TILE_PART_MODE (set by the build):
// the kernels of dcn4_kernels.hip instantiated in a translation unit of their
// own, so that the pairs compile in parallel.  The kernels and their
// citations are in dcn4_kernels.hip.
#if !defined(DCN4_TILE_PART_DT) || !defined(DCN4_TILE_PART_MODE)
#error "dcn4_tile_part.hip is built once per pair with -DDCN4_TILE_PART_DT=d -DDCN4_TILE_PART_MODE=m"
#endif
#include "dcn4_kernels.hip"
