// The fp8-KV kernel again, reading KV through a page table (separate
// instantiations in their own translation unit; see fp8_decode.hip).
#define MLA_PAGED_KV
#include "fp8_decode.hip"
