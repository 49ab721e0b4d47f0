// The library's e4m3 decode kernels (mla_decode_kernel<1, PH>) with one
// change: the query fragments are forced resident in VGPRs right after their
// loads, before any copy is issued.  Without it the compiler's wait-count
// pass, which does not see the inline-assembly copies, keeps the 36 query
// loads pending into the key loop and waits for them there (vmcnt 35 down to
// 9 across the QK step); at run time those literals also count the copies of
// the rounds issued ahead, so each step waits for the next round to land and
// the four-round ring prefetches about one round.  Everything else is the
// validated source, compiled a second time under other names, so the
// library's own kernels keep their machine code.  Chosen only when
// MLA_DECODE_KERNEL=qres, for e4m3 caches.
#define MLA_DECODE_Q_RESIDENT 1
#define mla_decode_kernel mla_decode_kernel_qres
#define mla_decode_kernel_pairs mla_decode_kernel_pairs_qres
#define launch_decode launch_decode_qres
#include "decode_kernel.hip"
