// Greedy verification for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops): the same kernel as mtp_verify, with its per-row
// argmax keys and per-sequence completion counters in a file-scope device array instead
// of a handle's workspace. No handle, no workspace, no allocation.
//
// The array is static device memory of the library's code object: each GPU the library
// runs on holds its own copy at its own address until the process ends. Host code never
// uses the array's name as an address (on the host it names a stand-in, not device
// memory): the device address is looked up once per device with hipGetSymbolAddress and
// kept, and only that pointer is handed to the kernels.
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "mtp.h"

namespace {

using namespace mtp;

constexpr int kNaMaxBatch = MTP_NOALLOC_MAX_BATCH;
constexpr int kNaMaxK = 100;
constexpr int kNaKeyStride = (kNaMaxK + 1 + kSeqLineU64 - 1) / kSeqLineU64 * kSeqLineU64;
constexpr size_t kNaKeyBytes = (size_t)kNaMaxBatch * kNaKeyStride * 8;
constexpr size_t kNaCounterBytes = (size_t)kNaMaxBatch * kSeqLineU32 * 4;
constexpr size_t kNaScratchBytes = kNaKeyBytes + kNaCounterBytes;  // 320 KiB
constexpr int kNaMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNaScratchBytes];

struct DeviceScratch {
  std::once_flag once;
  hipError_t status = hipErrorNotInitialized;
  char* ptr = nullptr;  // device address of `scratch` on this device
};
DeviceScratch g_scratch[kNaMaxDevices];

// Device address of this device's copy of `scratch` (looked up on the first call made with
// the device current), or null when the lookup failed.
char* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kNaMaxDevices) return nullptr;
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&] {
    void* p = nullptr;
    d.status = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d.status == hipSuccess) d.ptr = static_cast<char*>(p);
  });
  return d.status == hipSuccess ? d.ptr : nullptr;
}

// Zero n 32-bit words (a kernel rather than hipMemsetAsync, so that the call can be
// captured into a graph).
__global__ void zero_words_kernel(uint32_t* p, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

extern "C" mtp_status mtp_verify_noalloc(const float* target_logits, const int32_t* draft_tokens,
                                         int32_t B, int32_t K, int32_t vocab,
                                         int32_t* accepted_len, int32_t* next_token,
                                         void* stream) {
  if (!target_logits || !accepted_len || !next_token) return MTP_ERR_INVALID_ARG;
  if (K > 0 && !draft_tokens) return MTP_ERR_INVALID_ARG;
  if (B < 1 || K < 0 || vocab < 1) return MTP_ERR_SHAPE;
  if (B > kNaMaxBatch || K > kNaMaxK) return MTP_ERR_CAPACITY;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MTP_ERR_HIP;
  char* base = scratch_ptr(dev);
  if (!base) return MTP_ERR_HIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int kstride = (K + 1 + kSeqLineU64 - 1) / kSeqLineU64 * kSeqLineU64;
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(base);
  unsigned* counters = reinterpret_cast<unsigned*>(base + kNaKeyBytes);
  // The keys and counters must start at zero; whatever an earlier call left is cleared.
  const long key_words = (long)B * kstride * 2, cnt_words = (long)B * kSeqLineU32;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((key_words + 255) / 256)), dim3(256), 0,
                     s, reinterpret_cast<uint32_t*>(keys), key_words);
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((cnt_words + 255) / 256)), dim3(256), 0,
                     s, reinterpret_cast<uint32_t*>(counters), cnt_words);
  if (hipGetLastError() != hipSuccess) return MTP_ERR_HIP;
  VerifyParams p{};
  p.logits = target_logits;
  p.draft = draft_tokens;
  p.K = K;
  p.V = vocab;
  p.keys = keys;
  p.kstride = kstride;
  p.counters = counters;
  p.accepted = accepted_len;
  p.next = next_token;
  return launch_verify(p, B, s) == hipSuccess ? MTP_OK : MTP_ERR_HIP;
}
