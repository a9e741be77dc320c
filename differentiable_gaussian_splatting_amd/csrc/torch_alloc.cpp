// torch_alloc.cpp -- allocator callbacks for gs_ctx_create that call
// PyTorch's HIP caching allocator from C, so that the library's allocations
// take the caching allocator's stream-ordered blocks (and show in its
// statistics) without a Python call per allocation.  Built as its own shared
// library against libc10_hip; libgsmi.so does not depend on it.
#include <c10/hip/HIPCachingAllocator.h>

#include <cstddef>

extern "C" {

// gs_alloc_fn: NULL when the allocator throws (out of memory)
void* gs_torch_alloc(void* user, size_t bytes, void* stream)
{
    (void)user;
    try {
        return c10::hip::HIPCachingAllocator::raw_alloc_with_stream(bytes, static_cast<hipStream_t>(stream));
    } catch (...) {
        return nullptr;
    }
}

// gs_free_fn
void gs_torch_free(void* user, void* ptr, size_t bytes, void* stream)
{
    (void)user;
    (void)bytes;
    (void)stream;
    try {
        c10::hip::HIPCachingAllocator::raw_delete(ptr);
    } catch (...) {
    }
}

}  // extern "C"
