// The main decode kernels for paged KV: the same source as kernels.hip,
// instantiated for a page-table source of KV rows (see launch_main_paged).
#define MLA_PAGED_KV 1
#include "kernels.hip"
