// The header seen by a C++ caller: it compiles under -Wall -Wextra -Werror, and its
// entry points keep C linkage (their addresses convert to pointers to C functions
// of the declared types).
#include "mxq.h"

extern "C" typedef mxq_status grouped_fn(const uint16_t*, int64_t, const int64_t*, int64_t, uint16_t, uint32_t,
                                         const mxq_sr*, const mxq_nvfp4_out*, const mxq_nvfp4_out*,
                                         const mxq_fp8_out*, void*, size_t, void*);
extern "C" typedef size_t size_fn(int64_t, int64_t, int64_t, uint32_t);

int main() {
    grouped_fn* g = &mxq_group_rht_quant_nvfp4;
    size_fn* q = &mxq_group_rht_quant_nvfp4_workspace_size;
    return (g != nullptr && q != nullptr) ? 0 : 1;
}
