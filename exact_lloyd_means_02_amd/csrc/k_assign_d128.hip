// FlashAssign, small-D kernel for 2-byte inputs at padded D = 128 (the headline width): the same
// source as k_assign.hip, built in a compilation unit of its own so that it can take the
// compiler's iterative ILP scheduling strategy (k_assign.hip takes the memory-clause strategy,
// under which the split-D kernel runs faster).  Only the kernel and its launcher are compiled here.
#define FKM_ASSIGN_D128_UNIT 1
#include "k_assign.hip"
