// sg_lib.hip -- single translation unit of libsg (gfx950).  Every kernel
// and the device error record live in one code object.
#include "sg_common.hip"
#include "sg_skiprs.hip"
#include "sg_partition.hip"
#include "sg_hhash.hip"
#include "sg_topk.hip"
#include "sg_dgc.hip"
#include "sg_merge.hip"
#include "sg_aggregate.hip"
#include "sg_encode.hip"
#include "sg_decode.hip"
#include "sg_statsw.hip"
#include "sg_stats.hip"
