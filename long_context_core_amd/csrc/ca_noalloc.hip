// The forward for callers that cannot allocate: ca_forward_noalloc.
//
// ca_forward and ca_forward_masked take a caller-allocated workspace and copy
// the host-built work queue into it through pinned staging buffers that the
// library grows with hipHostMalloc.  Code under graph capture, tight serving
// loops and harnesses that forbid allocation can do neither.  This entry point
// runs the same queue and the same kernels with the queue held in `scratch`, a
// fixed device array of this library (one per GPU, for the life of the
// process), and moves the queue bytes by value in the arguments of small store
// kernels: no device or pinned allocation, no host buffer that must outlive the
// call, and a captured graph replays the stores with the bytes of the call.

#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <vector>

#include "ca_internal.h"

namespace {

// Queue and decode staging of one call.  Device address: g_scratch_ptr[dev]
// (hipGetSymbolAddress); in host code the name `scratch` is only a stand-in
// for the symbol and is never used as a pointer.
static __device__ __align__(256) unsigned char scratch[CA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array, looked up once per device
// with that device current.
ca_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ca::set_error(CA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return ca::set_error(CA_ERR_UNSUPPORTED, "device index %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return ca::set_error(CA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CA_OK;
}

// Queue bytes travel by value in the kernel arguments: 3,072 bytes per launch
// keeps the explicit arguments (with the offset and count) well inside the
// 4 KiB the runtime takes for every kernel.
constexpr uint32_t kStoreWords = 768;
struct StoreChunk {
  uint64_t offset;           // byte offset in the destination, a multiple of 4
  uint32_t n_words;          // <= kStoreWords
  uint32_t pad;
  uint32_t words[kStoreWords];
};

__global__ void __launch_bounds__(256) store_words_kernel(uint32_t* dst, StoreChunk c) {
  uint32_t* d = dst + c.offset / 4;
  for (uint32_t i = threadIdx.x; i < c.n_words; i += 256) d[i] = c.words[i];
}

}  // namespace

extern "C" ca_status ca_forward_noalloc(const ca_shape* shape, const ca_task* tasks_host,
                                        const ca_task_mask* masks_host, int32_t n_tasks, const void* Q,
                                        const void* K, const void* V, void* O, float* LSE, void* stream) {
  ca::PreparedFwd pf;
  std::vector<char> host;
  size_t need = 0;
  const void* tensors[5] = {Q, K, V, O, LSE};
  ca_status st = ca::build_forward_queue(shape, tasks_host, masks_host, n_tasks, nullptr, tensors, pf, host, &need);
  if (st != CA_OK) return st;
  if (pf.n_items == 0 && pf.n_dec_items == 0) return CA_OK;
  if (need > (size_t)CA_NOALLOC_SCRATCH_BYTES)
    return ca::set_error(CA_ERR_WORKSPACE,
                         "the call needs %zu bytes of scratch; ca_forward_noalloc holds at most %zu "
                         "(use ca_forward_masked with a workspace)",
                         need, (size_t)CA_NOALLOC_SCRATCH_BYTES);
  void* base = nullptr;
  st = scratch_of_current_device(&base);
  if (st != CA_OK) return st;
  pf.ws = base;
  hipStream_t hs = (hipStream_t)stream;
  const size_t n_words = host.size() / 4;     // the queue layout is 256-byte aligned
  StoreChunk c;
  for (size_t w0 = 0; w0 < n_words; w0 += kStoreWords) {
    c.offset = (uint64_t)w0 * 4;
    c.n_words = (uint32_t)std::min<size_t>(kStoreWords, n_words - w0);
    c.pad = 0;
    std::memcpy(c.words, host.data() + w0 * 4, (size_t)c.n_words * 4);
    hipLaunchKernelGGL(store_words_kernel, dim3(1), dim3(256), 0, hs, (uint32_t*)base, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return ca::set_error(CA_ERR_HIP, "queue store launch: %s", hipGetErrorString(e));
  }
  return ca::launch_prepared_forward(pf, Q, K, V, O, LSE, stream);
}
