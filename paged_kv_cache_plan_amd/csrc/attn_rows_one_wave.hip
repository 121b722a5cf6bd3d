// The paged row kernel with one wave per workgroup: attn_rows.hip compiled a
// second time with PKV_ROWS_WAVES = 1, as a translation unit of its own so
// that both sets of kernels build in parallel.  Decode plans whose work items
// average a few 16-key blocks use it (see attn_rows.hip).
#define PKV_ROWS_WAVES 1
#include "attn_rows.hip"
