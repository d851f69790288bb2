// FlashAssign, small-D kernel for 2-byte inputs at padded D = 64: the same source as
// k_assign.hip, built in a compilation unit of its own so that it can take the compiler's
// default scheduling strategy (the build gives k_assign.hip the memory-clause strategy, which is
// the faster one at the other widths).  Only the kernel and its launcher are compiled here.
#define FKM_ASSIGN_D64_UNIT 1
#include "k_assign.hip"
