// The library's read-only device tables, generated when the library is built
// (e8q_tablegen.cpp, layout in e8q_tables_index.h) and embedded in the device
// code object: every GPU that loads the library holds its own copy from load
// time on, so no entry point allocates, uploads or waits for a table.
#include <hip/hip_runtime.h>

#include <mutex>

#include "e8q_tables_index.h"

namespace e8q {

// Not const, and marked used: the device compiler drops a const device
// variable that no kernel of this file reads, and the runtime then has no
// symbol to resolve.  Kernels only read it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wc23-extensions"
__device__ __attribute__((used, aligned(256))) unsigned char g_table_blob[] = {
#embed "e8q_tables.bin"
};
#pragma clang diagnostic pop

static_assert(sizeof(g_table_blob) == gen::kBlobBytes, "table blob size");

// Device address of the blob on the current device (looked up once per
// device; a host-side query, nothing is enqueued).
const unsigned char* table_blob_address() {
    static std::mutex mu;
    static const unsigned char* addr[64] = {nullptr};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_table_blob)) != hipSuccess) return nullptr;
        addr[dev] = static_cast<const unsigned char*>(p);
    }
    return addr[dev];
}

}  // namespace e8q
