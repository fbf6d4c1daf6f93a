// Accept / resample without a context and without any allocation, for callers
// that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid it).  It runs the kernels of uno_accept; what
// uno_accept keeps in the context's workspace (the row descriptors of the
// resample draws, the chunk sums of the integer CDF, the accept lengths and the
// drawn tokens) lives here in one file-scope device array per GPU.
//
// Every call on a GPU shares that GPU's array and leaves its contents behind:
// calls that overlap on one GPU (two streams, two threads) race.  Nothing in the
// array has to start at zero: each call writes every word it reads first.
#include <mutex>

#include "../../include/uno.h"
#include "uno_internal.h"

namespace {

constexpr int kNaMaxSeqs = 1024;              // sequences per call
constexpr int kNaMaxChunks = 128;             // CDF chunks per row: vocab <= 128 * 2048
constexpr size_t kNaDesc = 0;                                        // RowDesc [n]
constexpr size_t kNaK = 40960;                                       // int32 [n]
constexpr size_t kNaZ = kNaK + 4 * kNaMaxSeqs;                       // int32 [n]
constexpr size_t kNaErr = kNaZ + 4 * kNaMaxSeqs;                     // int32 (unused flags)
constexpr size_t kNaChunks = kNaErr + 256;                           // uint64 [n, chunks]
constexpr size_t kNaBytes = kNaChunks + 8 * (size_t)kNaMaxSeqs * kNaMaxChunks;
static_assert(sizeof(RowDesc) * kNaMaxSeqs <= kNaK, "descriptor room");
static_assert(kNaChunks % 256 == 0, "aligned chunk sums");

}  // namespace

// 1.05 MiB per GPU, held until the process ends.  In host code this name is a
// stand-in, not a device address: the kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kNaBytes];

namespace {

constexpr int kNaMaxDevices = 64;
std::mutex g_na_mu;
unsigned char* g_na_ptr[kNaMaxDevices] = {};

// Device address of this GPU's scratch array (looked up once per device, with
// that device current).
hipError_t scratch_of_current(unsigned char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kNaMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_na_mu);
  if (!g_na_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_na_ptr[dev] = static_cast<unsigned char*>(p);
  }
  *out = g_na_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t noalloc_prime() {
  unsigned char* p = nullptr;
  return scratch_of_current(&p);
}

extern "C" uno_status uno_accept_noalloc(uint64_t seed, int32_t n, int32_t block_size,
                                         int32_t vocab, const float* d_p, const float* d_q,
                                         const int32_t* d_draft, const int32_t* d_seq_ids,
                                         const int32_t* d_pos, const int32_t* d_iter,
                                         int32_t* d_out, int32_t* d_n_out, int32_t* d_err,
                                         void* stream) {
  if (n < 1 || n > kNaMaxSeqs)
    return (uno_status)uno_fail_global(UNO_ERR_INVALID_ARG,
                                       "accept_noalloc: n must be in 1..1024 (the static scratch holds 1024 sequences)");
  if (block_size < 1 || block_size > 64)
    return (uno_status)uno_fail_global(UNO_ERR_INVALID_ARG, "accept_noalloc: block_size must be in 1..64");
  if (vocab < 2 || vocab > kNaMaxChunks * CDF_CHUNK)
    return (uno_status)uno_fail_global(UNO_ERR_INVALID_ARG,
                                       "accept_noalloc: vocab must be in 2..262144 (the static scratch holds 128 CDF chunks per row)");
  if (!d_p || !d_draft || !d_seq_ids || !d_pos || !d_iter || !d_out || !d_n_out ||
      (!d_q && block_size > 1))
    return (uno_status)uno_fail_global(UNO_ERR_INVALID_ARG, "accept_noalloc: null buffer");
  unsigned char* base = nullptr;
  hipError_t e = scratch_of_current(&base);
  if (e != hipSuccess)
    return (uno_status)uno_fail_global(UNO_ERR_DEVICE, hipGetErrorString(e));
  hipStream_t s = static_cast<hipStream_t>(stream);
  RowDesc* desc = reinterpret_cast<RowDesc*>(base + kNaDesc);
  int32_t* acc_k = reinterpret_cast<int32_t*>(base + kNaK);
  int32_t* acc_z = reinterpret_cast<int32_t*>(base + kNaZ);
  int32_t* err = d_err ? d_err : reinterpret_cast<int32_t*>(base + kNaErr);
  uint64_t* chunk_tot = reinterpret_cast<uint64_t*>(base + kNaChunks);
  const int B = block_size, V = vocab;
  if ((e = launch_accept_test(seed, n, B, V, d_p, d_q, B - 1, d_draft, d_seq_ids, d_pos, d_iter,
                              acc_k, acc_z, desc, err, s)) != hipSuccess ||
      (e = launch_cdf(desc, n, V, chunk_tot, err, s)) != hipSuccess ||
      (e = launch_accept_commit(n, B, d_draft, acc_k, acc_z, d_seq_ids, d_out, d_n_out, nullptr,
                                nullptr, nullptr, s)) != hipSuccess)
    return (uno_status)uno_fail_global(UNO_ERR_DEVICE, hipGetErrorString(e));
  return UNO_OK;
}
