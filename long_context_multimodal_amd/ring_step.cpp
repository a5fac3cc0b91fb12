// mmsp_ring_step: one rank's MM-SP training step through the C-ABI alone.
//
// A caller without Python: device memory from hipMalloc, the default stream,
// and the library's entry points for the whole path -- zigzag shard balance,
// the ring forward over every resident chunk with the fused merge and the
// bf16 output, the backward preprocess and the ring backward.
//
//   mmsp_ring_step IN OUT
//
// IN (little-endian): int32 header[8] = {0x4d4d5350, n_tokens, n_ranks, rank,
//   hq, hkv, d, causal}, then bf16 bits of q [shard][hq][d], k and v
//   [n_ranks][shard][hkv][d] (chunk c holds the keys of rank c's shard),
//   dout [shard][hq][d], with shard = n_tokens / n_ranks.
// OUT: bf16 o [shard][hq][d], fp32 lse [hq][shard], dq [shard][hq][d],
//   dk and dv [n_ranks][shard][hkv][d].
// Exit status 0 on success; otherwise a message on stderr and status 1.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../include/mmsp.h"

namespace {

[[noreturn]] void fail(const char* what, const char* detail) {
  std::fprintf(stderr, "mmsp_ring_step: %s: %s\n", what, detail);
  std::exit(1);
}

void hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) fail(what, hipGetErrorString(e));
}

void mmsp_ok(int status, const char* what) {
  if (status != MMSP_OK) fail(what, mmsp_status_string(status));
}

template <typename T>
T* device_copy(const std::vector<T>& host) {
  T* p = nullptr;
  hip_ok(hipMalloc((void**)&p, host.size() * sizeof(T)), "hipMalloc");
  hip_ok(hipMemcpy(p, host.data(), host.size() * sizeof(T), hipMemcpyHostToDevice), "hipMemcpy");
  return p;
}

template <typename T>
T* device_alloc(size_t n) {
  T* p = nullptr;
  hip_ok(hipMalloc((void**)&p, n * sizeof(T)), "hipMalloc");
  return p;
}

template <typename T>
void read_into(std::FILE* f, std::vector<T>& v) {
  if (std::fread(v.data(), sizeof(T), v.size(), f) != v.size()) fail("input", "file too short");
}

template <typename T>
void write_from(std::FILE* f, const T* dev, size_t n) {
  std::vector<T> host(n);
  hip_ok(hipMemcpy(host.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost), "hipMemcpy");
  if (std::fwrite(host.data(), sizeof(T), n, f) != n) fail("output", "write failed");
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) fail("usage", "mmsp_ring_step IN OUT");
  std::FILE* in = std::fopen(argv[1], "rb");
  if (!in) fail("input", "cannot open");
  int32_t h[8];
  if (std::fread(h, sizeof(int32_t), 8, in) != 8 || h[0] != 0x4d4d5350) fail("input", "bad header");
  const int32_t n = h[1], p = h[2], rank = h[3], hq = h[4], hkv = h[5], d = h[6];
  const bool causal = h[7] != 0;
  if (n <= 0 || p <= 0 || n % (2 * p) != 0 || hq <= 0 || hkv <= 0 || d <= 0)
    fail("input", "bad sizes");
  const size_t shard = (size_t)n / p;
  const size_t q_elems = shard * hq * d, kv_elems = shard * hkv * d;
  std::vector<uint16_t> q(q_elems), k(kv_elems * p), v(kv_elems * p), dout(q_elems);
  read_into(in, q);
  read_into(in, k);
  read_into(in, v);
  read_into(in, dout);
  std::fclose(in);

  uint16_t* dq_in = device_copy(q);
  uint16_t* dk_in = device_copy(k);
  uint16_t* dv_in = device_copy(v);
  uint16_t* d_dout = device_copy(dout);
  int32_t* perm = device_alloc<int32_t>(n);
  float* o = device_alloc<float>(q_elems);
  float* lse = device_alloc<float>((size_t)hq * shard);
  uint16_t* o16 = device_alloc<uint16_t>(q_elems);
  float* delta = device_alloc<float>((size_t)hq * shard);
  float* dq = device_alloc<float>(q_elems);
  float* dk = device_alloc<float>(kv_elems * p);
  float* dv = device_alloc<float>(kv_elems * p);

  // shard balance: zigzag needs no labels and no workspace
  mmsp_ok(mmsp_shard_balance(nullptr, n, p, MMSP_BALANCE_ZIGZAG, 0, perm, nullptr, nullptr, 0,
                             nullptr),
          "mmsp_shard_balance");
  std::vector<const void*> ks(p), vs(p);
  std::vector<const int32_t*> kps(p);
  std::vector<float*> dks(p), dvs(p);
  for (int c = 0; c < p; ++c) {
    ks[c] = dk_in + c * kv_elems;
    vs[c] = dv_in + c * kv_elems;
    kps[c] = perm + c * shard;
    dks[c] = dk + c * kv_elems;
    dvs[c] = dv + c * kv_elems;
  }
  const int32_t* q_pos = perm + rank * shard;
  const float scale = (float)(1.0 / std::sqrt((double)d));
  const uint32_t flags = causal ? MMSP_CAUSAL : 0u;
  mmsp_ok(mmsp_ring_forward(dq_in, ks.data(), vs.data(), q_pos, kps.data(), nullptr, p, rank,
                            (int32_t)shard, (int32_t)shard, hq, hkv, d, scale, flags, o, lse, o16,
                            nullptr),
          "mmsp_ring_forward");
  mmsp_ok(mmsp_ring_backward(dq_in, ks.data(), vs.data(), d_dout, o16, lse, q_pos, kps.data(),
                             nullptr, p, rank, (int32_t)shard, (int32_t)shard, hq, hkv, d, scale,
                             flags, delta, dq, dks.data(), dvs.data(), nullptr),
          "mmsp_ring_backward");
  hip_ok(hipDeviceSynchronize(), "step");

  std::FILE* out = std::fopen(argv[2], "wb");
  if (!out) fail("output", "cannot open");
  write_from(out, o16, q_elems);
  write_from(out, lse, (size_t)hq * shard);
  write_from(out, dq, q_elems);
  write_from(out, dk, kv_elems * p);
  write_from(out, dv, kv_elems * p);
  std::fclose(out);
  for (void* ptr : {(void*)dq_in, (void*)dk_in, (void*)dv_in, (void*)d_dout, (void*)perm,
                    (void*)o, (void*)lse, (void*)o16, (void*)delta, (void*)dq, (void*)dk,
                    (void*)dv})
    hip_ok(hipFree(ptr), "hipFree");
  return 0;
}
