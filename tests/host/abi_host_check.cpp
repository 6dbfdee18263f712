// Host-only check of the C ABI: argument validation, workspace plans and
// launch configurations, run on the CPU with no GPU.
//
// The library's sources are compiled host-only (kernel bodies are not built)
// with -DDSA_DEBUG and address/undefined-behaviour sanitizers, and linked
// with this file, which stands in for the few HIP runtime calls the host side
// makes: device query, LDS attribute, launch configuration and kernel launch.
// A "launch" only records its configuration and checks it against the
// device's limits; no device pointer is ever dereferenced on the host, so
// buffers are fake aligned addresses.
//
// Every entry point is called with
//   * invalid arguments: the documented status, and nothing launched;
//   * valid arguments over the supported shapes: DSA_OK, at least one launch,
//     every launch within the grid, block and LDS limits, and the plan
//     checks compiled in by DSA_DEBUG (workspace carve-ups) all holding;
//   * one byte less workspace than the size query reports: DSA_ERR_WORKSPACE.
// Exit status 0 when every check holds; a failure prints its line.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>

#include "dsa.h"

// ---- stand-ins for the HIP runtime's host entry points ---------------------

namespace {
struct LaunchCfg {
  dim3 grid, block;
  size_t lds;
  hipStream_t stream;
};
LaunchCfg g_cfg;
int g_launches = 0;
int g_bad_launches = 0;
int g_device = 0;  // the device hipGetDevice reports
const char* g_arch[2] = {"gfx950:sramecc+:xnack-", "gfx942:sramecc+:xnack-"};
// function-local maps: the library's module constructors register kernels
// before this file's globals would be constructed
std::map<const void*, std::string>& names() {
  static std::map<const void*, std::string> m;
  return m;
}
std::map<const void*, int>& lds_limits() {  // dynamic LDS opted in per kernel
  static std::map<const void*, int> m;
  return m;
}
std::map<const void*, size_t>& vars() {  // registered device variables and their sizes
  static std::map<const void*, size_t> m;
  return m;
}
int g_symbol_lookups = 0;
constexpr int kMaxGrid[3] = {2147483647, 65536, 65536};
constexpr size_t kLdsPerCu = 160 * 1024;
constexpr size_t kLdsDefault = 64 * 1024;
}  // namespace

extern "C" {
void** __hipRegisterFatBinary(const void*) {
  static void* handle = nullptr;
  return &handle;
}
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterFunction(void**, const void* host_fn, char*, const char* name, unsigned, uint3*, uint3*, dim3*,
                           dim3*, int*) {
  names()[host_fn] = name;
}
hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t lds, hipStream_t st) {
  g_cfg = LaunchCfg{grid, block, lds, st};
  return hipSuccess;
}
hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* lds, hipStream_t* st) {
  *grid = g_cfg.grid;
  *block = g_cfg.block;
  *lds = g_cfg.lds;
  *st = g_cfg.stream;
  return hipSuccess;
}
hipError_t hipLaunchKernel(const void* fn, dim3 grid, dim3 block, void**, size_t lds, hipStream_t) {
  ++g_launches;
  const std::string name = names().count(fn) ? names()[fn] : std::string("?");
  const unsigned g[3] = {grid.x, grid.y, grid.z};
  bool ok = block.x >= 1 && block.x * block.y * block.z <= 1024 && block.x % 64 == 0;
  for (int i = 0; i < 3; ++i) ok = ok && g[i] >= 1 && g[i] <= (unsigned)kMaxGrid[i];
  const size_t limit = lds_limits().count(fn) ? (size_t)lds_limits()[fn] : kLdsDefault;
  ok = ok && lds <= limit && lds <= kLdsPerCu;
  if (!ok) {
    ++g_bad_launches;
    std::fprintf(stderr, "bad launch of %s: grid (%u, %u, %u) block (%u, %u, %u) lds %zu (limit %zu)\n",
                 name.c_str(), grid.x, grid.y, grid.z, block.x, block.y, block.z, lds, limit);
  }
  return hipSuccess;
}
void __hipRegisterVar(void**, void* var, char*, const char* name, int, size_t size, int, int) {
  vars()[var] = size;
  (void)name;
}
// the device copy of a registered variable lives at a fake device address
hipError_t hipGetSymbolAddress(void** dev_ptr, const void* symbol) {
  if (!vars().count(symbol)) return hipErrorInvalidSymbol;
  *dev_ptr = (void*)((uintptr_t)1 << 44);
  ++g_symbol_lookups;
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipGetDevice(int* d) {
  *d = g_device;
  return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* p, int d) {
  std::memset(p, 0, sizeof(*p));
  std::snprintf(p->gcnArchName, sizeof(p->gcnArchName), "%s", g_arch[d == 1]);
  p->maxThreadsPerBlock = 1024;
  for (int i = 0; i < 3; ++i) p->maxGridSize[i] = kMaxGrid[i];
  p->multiProcessorCount = 256;
  p->sharedMemPerBlock = kLdsDefault;
  p->sharedMemPerBlockOptin = kLdsPerCu;
  return hipSuccess;
}
hipError_t hipFuncSetAttribute(const void* fn, hipFuncAttribute attr, int value) {
  if (attr == hipFuncAttributeMaxDynamicSharedMemorySize) {
    if (value < 0 || (size_t)value > kLdsPerCu) return hipErrorInvalidValue;
    lds_limits()[fn] = value;
  }
  return hipSuccess;
}
}  // extern "C"

// ---- checks ------------------------------------------------------------------

namespace {
int g_failures = 0;
int g_checks = 0;

void expect(bool ok, const char* what, int line) {
  ++g_checks;
  if (!ok) {
    ++g_failures;
    std::fprintf(stderr, "FAIL line %d: %s\n", line, what);
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// a call that must return `want`; it launches iff want == DSA_OK and `launches`
#define CALL(want, launches, call)                                                                           \
  do {                                                                                                       \
    const int before = g_launches, bad_before = g_bad_launches;                                              \
    const dsa_status_t got = (call);                                                                         \
    ++g_checks;                                                                                              \
    const bool launched = g_launches > before;                                                               \
    if (got != (want) || launched != (launches) || g_bad_launches != bad_before) {                           \
      ++g_failures;                                                                                          \
      std::fprintf(stderr, "FAIL line %d: %s -> %d (%s), want %d; launched %d\n", __LINE__, #call, (int)got, \
                   dsa_status_str(got), (int)(want), (int)launched);                                         \
    }                                                                                                        \
  } while (0)

// fake device addresses: never dereferenced on the host
void* dptr(uintptr_t slot) { return (void*)(uintptr_t)((uintptr_t)1 << 40 | slot << 30); }
void* const kWs = dptr(1);
void* const kMisaligned = (void*)((char*)dptr(2) + 8);
const float kNaN = __builtin_nanf("");

// ---- per entry point ---------------------------------------------------------

void check_misc() {
  EXPECT(dsa_abi_version() == DSA_ABI_VERSION);
  for (int s = 0; s <= 7; ++s) EXPECT(dsa_status_str((dsa_status_t)s) != nullptr);
}

void check_fold() {
  void *q = dptr(3), *w = dptr(4), *o = dptr(5);
  float *qs = (float*)dptr(6), *os = (float*)dptr(7);
  CALL(DSA_OK, true, dsa_fold_index_query(q, qs, DSA_FP8_E4M3, w, DSA_BF16, 131072, o, os, nullptr));
  CALL(DSA_OK, true, dsa_fold_index_query(q, qs, DSA_FP8_E4M3, w, DSA_F32, 64, o, os, nullptr));
  CALL(DSA_OK, true, dsa_fold_index_query(q, nullptr, DSA_F32, w, DSA_F32, 512, o, nullptr, nullptr));
  CALL(DSA_OK, true, dsa_fold_index_query(q, qs, DSA_FP8_E4M3, w, DSA_BF16, 1, o, os, nullptr));
  CALL(DSA_OK, false, dsa_fold_index_query(nullptr, nullptr, DSA_FP8_E4M3, nullptr, DSA_BF16, 0, nullptr,
                                           nullptr, nullptr));
  CALL(DSA_ERR_SHAPE, false, dsa_fold_index_query(q, qs, DSA_FP8_E4M3, w, DSA_BF16, -1, o, os, nullptr));
  CALL(DSA_ERR_DTYPE, false, dsa_fold_index_query(q, qs, DSA_BF16, w, DSA_BF16, 8, o, os, nullptr));
  CALL(DSA_ERR_DTYPE, false, dsa_fold_index_query(q, qs, DSA_F32, w, DSA_BF16, 8, o, os, nullptr));
  CALL(DSA_ERR_DTYPE, false, dsa_fold_index_query(q, qs, DSA_FP8_E4M3, w, DSA_FP8_E4M3, 8, o, os, nullptr));
  CALL(DSA_ERR_NULL, false, dsa_fold_index_query(nullptr, qs, DSA_FP8_E4M3, w, DSA_BF16, 8, o, os, nullptr));
  CALL(DSA_ERR_NULL, false, dsa_fold_index_query(q, nullptr, DSA_FP8_E4M3, w, DSA_BF16, 8, o, os, nullptr));
  CALL(DSA_ERR_NULL, false, dsa_fold_index_query(q, qs, DSA_FP8_E4M3, w, DSA_BF16, 8, o, nullptr, nullptr));
  CALL(DSA_ERR_NULL, false, dsa_fold_index_query(q, qs, DSA_FP8_E4M3, nullptr, DSA_BF16, 8, o, os, nullptr));
}

void check_scores() {
  void *qf = dptr(3), *k = dptr(4);
  float *qs = (float*)dptr(5), *ks = (float*)dptr(6), *out = (float*)dptr(7);
  const int64_t p64 = (int64_t)1 << 20;
  struct {
    int64_t T, S, rb, re, ld;
  } ok[] = {{1, 1, 0, 1, 1},        {512, 512, 0, 512, 512},   {8192, 8192, 100, 8192, 8200},
            {131072, 131072, 131071, 131072, 131072},          {p64, 64, 0, p64, 64},
            {p64, p64, p64 - 1000, p64, p64},                  {3, 1 << 30, 0, 3, 1 << 30},
            {(int64_t)1 << 23, 64, 0, (int64_t)1 << 23, 64}};   // more row blocks than a grid's y extent
  for (auto& c : ok) {
    CALL(DSA_OK, true, dsa_index_scores(qf, qs, k, ks, DSA_FP8_E4M3, c.T, c.S, nullptr, c.rb, c.re, out, c.ld,
                                        nullptr));
    CALL(DSA_OK, true, dsa_index_scores(qf, nullptr, k, nullptr, DSA_F32, c.T, c.S, nullptr, c.rb, c.re, out,
                                        c.ld, nullptr));
  }
  CALL(DSA_OK, false, dsa_index_scores(qf, qs, k, ks, DSA_FP8_E4M3, 8, 8, nullptr, 3, 3, out, 8, nullptr));
  CALL(DSA_OK, false, dsa_index_scores(qf, qs, k, ks, DSA_FP8_E4M3, 8, 0, nullptr, 0, 8, out, 0, nullptr));
  CALL(DSA_ERR_SHAPE, false, dsa_index_scores(qf, qs, k, ks, DSA_FP8_E4M3, 8, 8, nullptr, 0, 8, out, 7, nullptr));
  CALL(DSA_ERR_SHAPE, false, dsa_index_scores(qf, qs, k, ks, DSA_FP8_E4M3, 8, 8, nullptr, 5, 4, out, 8, nullptr));
  CALL(DSA_ERR_SHAPE, false, dsa_index_scores(qf, qs, k, ks, DSA_FP8_E4M3, 8, 8, nullptr, 0, 9, out, 8, nullptr));
  CALL(DSA_ERR_SHAPE, false, dsa_index_scores(qf, qs, k, ks, DSA_FP8_E4M3, 8, 8, nullptr, -1, 8, out, 8, nullptr));
  CALL(DSA_ERR_SHAPE, false, dsa_index_scores(kMisaligned, qs, k, ks, DSA_FP8_E4M3, 8, 8, nullptr, 0, 8, out, 8,
                                              nullptr));
  CALL(DSA_ERR_DTYPE, false, dsa_index_scores(qf, qs, k, ks, DSA_BF16, 8, 8, nullptr, 0, 8, out, 8, nullptr));
  CALL(DSA_ERR_NULL, false, dsa_index_scores(qf, nullptr, k, ks, DSA_FP8_E4M3, 8, 8, nullptr, 0, 8, out, 8,
                                             nullptr));
  CALL(DSA_ERR_NULL, false, dsa_index_scores(qf, qs, k, ks, DSA_FP8_E4M3, 8, 8, nullptr, 0, 8, nullptr, 8,
                                             nullptr));
}

void check_topk() {
  const float* sc = (const float*)dptr(3);
  int32_t *idx = (int32_t*)dptr(4), *cnt = (int32_t*)dptr(5);
  const int64_t* pos = (const int64_t*)dptr(6);
  struct {
    int64_t T, S, k;
  } ok[] = {{1, 1, 1},        {64, 100, 1},      {64, 5000, 64},      {48, 8192, 2048},   {40, 4000, 4096},
            {8, 131072, 2048}, {511, 16384, 2048}, {512, 16384, 2048}, {4, 300000, 4096}, {2, 1 << 21, 2048},
            {131072, 131072, 2048}};
  for (auto& c : ok) {
    const size_t ws = dsa_topk_workspace_size(c.T, c.S, c.k);
    CALL(DSA_OK, true, dsa_topk(sc, c.S, c.T, c.S, nullptr, c.k, idx, cnt, ws ? kWs : nullptr, ws, nullptr));
    CALL(DSA_OK, true, dsa_topk(sc, c.S + 3, c.T, c.S, pos, c.k, idx, nullptr, ws ? kWs : nullptr, ws, nullptr));
    CALL(DSA_OK, true, dsa_topk_dynamic(sc, c.S, c.T, c.S, nullptr, c.k, c.k / 2, 0.5f, idx, cnt,
                                        ws ? kWs : nullptr, ws, nullptr));
    if (ws) {
      CALL(DSA_ERR_WORKSPACE, false, dsa_topk(sc, c.S, c.T, c.S, nullptr, c.k, idx, cnt, kWs, ws - 1, nullptr));
      CALL(DSA_ERR_WORKSPACE, false, dsa_topk(sc, c.S, c.T, c.S, nullptr, c.k, idx, cnt, kMisaligned, ws, nullptr));
      CALL(DSA_ERR_WORKSPACE, false, dsa_topk(sc, c.S, c.T, c.S, nullptr, c.k, idx, cnt, nullptr, ws, nullptr));
    }
  }
  CALL(DSA_OK, false, dsa_topk(sc, 8, 0, 8, nullptr, 4, idx, cnt, nullptr, 0, nullptr));
  CALL(DSA_ERR_SHAPE, false, dsa_topk(sc, 8, 4, 8, nullptr, 0, idx, cnt, nullptr, 0, nullptr));
  CALL(DSA_ERR_SHAPE, false, dsa_topk(sc, 8, 4, 8, nullptr, DSA_MAX_TOPK + 1, idx, cnt, nullptr, 0, nullptr));
  CALL(DSA_ERR_SHAPE, false, dsa_topk(sc, 7, 4, 8, nullptr, 4, idx, cnt, nullptr, 0, nullptr));
  CALL(DSA_ERR_SHAPE, false, dsa_topk(sc, 8, -1, 8, nullptr, 4, idx, cnt, nullptr, 0, nullptr));
  CALL(DSA_ERR_NULL, false, dsa_topk(sc, 8, 4, 8, nullptr, 4, nullptr, cnt, nullptr, 0, nullptr));
  CALL(DSA_ERR_NULL, false, dsa_topk(nullptr, 8, 4, 8, nullptr, 4, idx, cnt, nullptr, 0, nullptr));
  CALL(DSA_ERR_SHAPE, false, dsa_topk_dynamic(sc, 8, 4, 8, nullptr, 4, 5, 0.f, idx, cnt, nullptr, 0, nullptr));
  CALL(DSA_ERR_SHAPE, false, dsa_topk_dynamic(sc, 8, 4, 8, nullptr, 4, -1, 0.f, idx, cnt, nullptr, 0, nullptr));
  CALL(DSA_ERR_SHAPE, false, dsa_topk_dynamic(sc, 8, 4, 8, nullptr, 4, 1, kNaN, idx, cnt, nullptr, 0, nullptr));
}

struct AttnShape {
  dsa_dtype_t dt;
  int64_t H, Dk, Dv;
  bool sep_v;
};
const AttnShape kAttnShapes[] = {{DSA_F32, 4, 64, 64, true},
                                 {DSA_BF16, 16, 128, 128, true},
                                 {DSA_BF16, 16, 128, 128, false},
                                 {DSA_BF16, 128, 576, 512, false},
                                 {DSA_BF16, 128, 576, 512, true}};

void check_attn() {
  void *q = dptr(3), *kv = dptr(4), *v = dptr(5), *out = dptr(6);
  const int32_t* idx = (const int32_t*)dptr(7);
  float* lse = (float*)dptr(8);
  const int64_t Ts[] = {1, 20, 64, 255, 256, 300, 131072};
  const int64_t ks[] = {1, 32, 33, 256, 2048, 3584, 4096};
  for (const AttnShape& s : kAttnShapes) {
    const int64_t ld_kv = s.Dk, ld_v = s.Dv;
    for (int64_t T : Ts) {
      for (int64_t k : ks) {
        const bool sup = true;  // every listed shape takes any k up to DSA_MAX_TOPK
        const size_t ws = dsa_sparse_attn_workspace_size(T, s.H, s.Dv, k, s.dt);
        const void* vv = s.sep_v ? v : nullptr;
        CALL(sup ? DSA_OK : DSA_ERR_UNSUPPORTED, sup,
             dsa_sparse_attn(q, T, s.H, s.Dk, s.dt, kv, ld_kv, vv, ld_v, s.Dv, 131072, idx, k, 0.05f, out,
                             (k & 1) ? lse : nullptr, ws ? kWs : nullptr, ws, nullptr));
        if (sup && ws) {
          CALL(DSA_ERR_WORKSPACE, false,
               dsa_sparse_attn(q, T, s.H, s.Dk, s.dt, kv, ld_kv, vv, ld_v, s.Dv, 131072, idx, k, 0.05f, out, lse,
                               kWs, ws - 1, nullptr));
        }
      }
    }
  }
  const AttnShape& m = kAttnShapes[3];
  auto mla = [&](int64_t T, int64_t H, dsa_dtype_t dt, const void* qq, int64_t ld_kv, int64_t S, int64_t k,
                 void* o) {
    return dsa_sparse_attn(qq, T, H, m.Dk, dt, kv, ld_kv, nullptr, 0, m.Dv, S, idx, k, 0.05f, o, nullptr, kWs,
                           (size_t)1 << 40, nullptr);
  };
  CALL(DSA_OK, true, mla(4, 128, DSA_BF16, q, 576, 3728270, 2048, out));   // 4 GiB of latent rows
  CALL(DSA_ERR_UNSUPPORTED, false, mla(4, 128, DSA_BF16, q, 576, 3728271, 2048, out));
  CALL(DSA_ERR_UNSUPPORTED, false, mla(4, 64, DSA_BF16, q, 576, 1000, 2048, out));
  CALL(DSA_ERR_DTYPE, false, mla(4, 128, DSA_FP8_E4M3, q, 576, 1000, 2048, out));
  CALL(DSA_ERR_SHAPE, false, mla(4, 128, DSA_BF16, q, 575, 1000, 2048, out));
  CALL(DSA_ERR_SHAPE, false, mla(4, 128, DSA_BF16, q, 580, 1000, 2048, out));      // ld not a multiple of 8
  CALL(DSA_ERR_SHAPE, false, mla(4, 128, DSA_BF16, q, 576, 0, 2048, out));
  CALL(DSA_ERR_SHAPE, false, mla(4, 128, DSA_BF16, q, 576, 1000, 0, out));
  CALL(DSA_ERR_SHAPE, false, mla(4, 128, DSA_BF16, q, 576, 1000, DSA_MAX_TOPK + 1, out));
  CALL(DSA_ERR_SHAPE, false, mla(4, 128, DSA_BF16, kMisaligned, 576, 1000, 2048, out));
  CALL(DSA_ERR_NULL, false, mla(4, 128, DSA_BF16, q, 576, 1000, 2048, nullptr));
  CALL(DSA_OK, false, mla(0, 128, DSA_BF16, nullptr, 576, 1000, 2048, nullptr));
}

void check_bwd() {
  void *q = dptr(3), *kv = dptr(4), *out = dptr(5), *dout = dptr(6), *dq = dptr(7);
  const int32_t* idx = (const int32_t*)dptr(8);
  const float* lse = (const float*)dptr(9);
  float* dkv = (float*)dptr(10);
  const int64_t Ts[] = {1, 37, 4100, 131072};
  const int64_t ks[] = {32, 256, 2048, 4096};
  for (int64_t T : Ts) {
    for (int64_t k : ks) {
      const size_t ws = dsa_sparse_attn_bwd_workspace_size(T, 128, k);
      CALL(DSA_OK, true, dsa_sparse_attn_bwd(q, T, 128, 576, DSA_BF16, kv, 576, 512, 131072, idx, k, 0.05f, out,
                                             lse, dout, dq, dkv, 576, kWs, ws, nullptr));
      CALL(DSA_ERR_WORKSPACE, false, dsa_sparse_attn_bwd(q, T, 128, 576, DSA_BF16, kv, 576, 512, 131072, idx, k,
                                                         0.05f, out, lse, dout, dq, dkv, 576, kWs, ws - 1, nullptr));
    }
  }
  auto bwd = [&](int64_t H, dsa_dtype_t dt, int64_t k, float* dk, int64_t ld_dkv) {
    return dsa_sparse_attn_bwd(q, 8, H, 576, dt, kv, 576, 512, 1000, idx, k, 0.05f, out, lse, dout, dq, dk, ld_dkv,
                               kWs, (size_t)1 << 40, nullptr);
  };
  CALL(DSA_ERR_UNSUPPORTED, false, bwd(128, DSA_F32, 256, dkv, 576));
  CALL(DSA_ERR_DTYPE, false, bwd(128, DSA_FP8_E4M3, 256, dkv, 576));
  CALL(DSA_ERR_UNSUPPORTED, false, bwd(64, DSA_BF16, 256, dkv, 576));
  CALL(DSA_ERR_UNSUPPORTED, false, bwd(128, DSA_BF16, 100, dkv, 576));
  CALL(DSA_ERR_SHAPE, false, bwd(128, DSA_BF16, 256, dkv, 500));
  CALL(DSA_ERR_NULL, false, bwd(128, DSA_BF16, 256, nullptr, 576));
}

void check_kl() {
  const float *qi = (const float*)dptr(3), *ki = (const float*)dptr(4), *w = (const float*)dptr(5);
  void *q = dptr(6), *kv = dptr(7);
  float *loss = (float*)dptr(8), *dqi = (float*)dptr(9), *dki = (float*)dptr(10), *dw = (float*)dptr(11);
  for (int64_t L : {1, 97, 600, 8192, 65536}) {
    const size_t ws = dsa_indexer_kl_workspace_size(L);
    CALL(DSA_OK, true, dsa_indexer_kl(qi, ki, w, q, 128, 576, DSA_BF16, kv, 576, L, 0.05f, loss, dqi, dki, dw, kWs,
                                      ws, nullptr));
    CALL(DSA_ERR_WORKSPACE, false, dsa_indexer_kl(qi, ki, w, q, 128, 576, DSA_BF16, kv, 576, L, 0.05f, loss, dqi,
                                                  dki, dw, kWs, ws - 1, nullptr));
  }
  EXPECT(dsa_indexer_kl_workspace_size(65537) == 0);
  CALL(DSA_ERR_UNSUPPORTED, false, dsa_indexer_kl(qi, ki, w, q, 128, 576, DSA_BF16, kv, 576, 65537, 0.05f, loss, dqi,
                                                  dki, dw, kWs, (size_t)1 << 40, nullptr));
  CALL(DSA_ERR_UNSUPPORTED, false, dsa_indexer_kl(qi, ki, w, q, 64, 576, DSA_BF16, kv, 576, 100, 0.05f, loss, dqi,
                                                  dki, dw, kWs, (size_t)1 << 40, nullptr));
  CALL(DSA_ERR_NULL, false, dsa_indexer_kl(qi, ki, w, q, 128, 576, DSA_BF16, kv, 576, 100, 0.05f, nullptr, dqi, dki,
                                           dw, kWs, (size_t)1 << 40, nullptr));
  CALL(DSA_OK, false, dsa_indexer_kl(qi, ki, w, q, 128, 576, DSA_BF16, kv, 576, 0, 0.05f, loss, dqi, dki, dw, nullptr,
                                     0, nullptr));
}

dsa_forward_args prefill_args(int64_t T, const AttnShape& s, bool fp8, int64_t k, int64_t q_offset, uint32_t flags) {
  dsa_forward_args a{};
  a.mode = DSA_MODE_PREFILL;
  a.flags = flags;
  a.T = T;
  a.idx_dtype = fp8 ? DSA_FP8_E4M3 : DSA_F32;
  a.q_idx = dptr(3);
  a.q_scale = fp8 ? (const float*)dptr(4) : nullptr;
  a.w_index = dptr(5);
  a.w_dtype = fp8 ? DSA_BF16 : DSA_F32;
  a.k_idx = dptr(6);
  a.k_scale = fp8 ? (const float*)dptr(7) : nullptr;
  a.attn_dtype = s.dt;
  a.q = dptr(8);
  a.H = s.H;
  a.Dk = s.Dk;
  a.Dv = s.Dv;
  a.kv = dptr(9);
  a.ld_kv = s.Dk;
  a.v = s.sep_v ? dptr(10) : nullptr;
  a.ld_v = s.Dv;
  a.topk = k;
  a.scale = 0.05f;
  a.q_offset = q_offset;
  a.dyn_theta = 0.3f;
  a.dyn_k_min = k / 8;
  return a;
}

void run_forward(const dsa_forward_args& a) {
  int32_t* idx = (int32_t*)dptr(11);
  void* out = dptr(12);
  const size_t ws = dsa_forward_workspace_size(&a);
  ++g_checks;
  if (ws == 0) {
    ++g_failures;
    std::fprintf(stderr, "FAIL: zero workspace for a valid forward (T %lld, mode %d)\n", (long long)a.T, a.mode);
    return;
  }
  CALL(DSA_OK, true, dsa_forward(&a, idx, out, kWs, ws, nullptr));
  CALL(DSA_OK, true, dsa_forward(&a, nullptr, out, kWs, ws, nullptr));
  // the size query covers the indices kept in the workspace (idx_out NULL)
  CALL(DSA_ERR_WORKSPACE, false, dsa_forward(&a, nullptr, out, kWs, ws - 1, nullptr));
  CALL(DSA_ERR_WORKSPACE, false, dsa_forward(&a, idx, out, kMisaligned, ws, nullptr));
  CALL(DSA_ERR_NULL, false, dsa_forward(&a, idx, nullptr, kWs, ws, nullptr));
}

void check_forward() {
  const uint32_t flag_sets[] = {0, DSA_FLAG_MATERIALIZE, DSA_FLAG_FUSED, DSA_FLAG_FUSED | DSA_FLAG_FORCE_FALLBACK,
                                DSA_FLAG_DYNAMIC_K, DSA_FLAG_DYNAMIC_K | DSA_FLAG_MATERIALIZE};
  // the tiny fp32 workload and short ragged prefills
  for (int64_t T : {1, 2, 300, 512, 777})
    for (uint32_t f : {0u, (uint32_t)DSA_FLAG_DYNAMIC_K}) run_forward(prefill_args(T, kAttnShapes[0], false, 64, 0, f));
  for (int64_t T : {1, 777, 4095, 4096, 6000, 8192})
    for (uint32_t f : flag_sets) {
      run_forward(prefill_args(T, kAttnShapes[1], true, 2048, 0, f));
      run_forward(prefill_args(T, kAttnShapes[3], true, 2048, 0, f));
    }
  for (int64_t T : {1000, 32768, 131072})
    for (uint32_t f : flag_sets) run_forward(prefill_args(T, kAttnShapes[3], true, 2048, 0, f));
  run_forward(prefill_args(5000, kAttnShapes[4], true, 3584, 0, 0));
  run_forward(prefill_args(300, kAttnShapes[3], true, 4096, 0, DSA_FLAG_FUSED));
  // chunks of a long prefill (the keys of the earlier chunks plus their own)
  const int64_t m20 = (int64_t)1 << 20;
  for (int64_t q0 : {(int64_t)1000, (int64_t)65536, m20 - 131072, m20 - 1000})
    for (uint32_t f : {0u, (uint32_t)DSA_FLAG_MATERIALIZE})
      run_forward(prefill_args(q0 == m20 - 1000 ? 1000 : 131072, kAttnShapes[3], true, 2048, q0, f));
  // batched decode over ragged caches
  struct {
    int64_t B, total, max_len;
  } dec[] = {{1, 1, 1}, {7, 9000, 3000}, {64, 4938934, 131072}, {4, 2244418, m20 + 64}, {64, 50000000, m20},
             {1000, 1000 * 2048, 4096}, {600, 600 * 70000, 131072},
             {70000, 70000 * 100, 100}};   // more sequences than a grid's y extent
  for (auto& d : dec) {
    for (uint32_t f : {0u, (uint32_t)DSA_FLAG_DYNAMIC_K}) {
      dsa_forward_args a = prefill_args(d.B, kAttnShapes[3], true, 2048, 0, f);
      a.mode = DSA_MODE_DECODE;
      a.seq_offsets = (const int64_t*)dptr(13);
      a.total_keys = d.total;
      a.max_len = d.max_len;
      run_forward(a);
    }
  }
  // invalid arguments
  int32_t* idx = (int32_t*)dptr(11);
  void* out = dptr(12);
  const size_t big = (size_t)1 << 40;
  CALL(DSA_ERR_NULL, false, dsa_forward(nullptr, idx, out, kWs, big, nullptr));
  EXPECT(dsa_forward_workspace_size(nullptr) == 0);
  dsa_forward_args a = prefill_args(100, kAttnShapes[3], true, 2048, 0, 0);
  CALL(DSA_OK, false, [&] { dsa_forward_args b = a; b.T = 0; return dsa_forward(&b, idx, nullptr, nullptr, 0, nullptr); }());
  auto bad = [&](dsa_status_t want, auto edit) {
    dsa_forward_args b = a;
    edit(b);
    CALL(want, false, dsa_forward(&b, idx, out, kWs, big, nullptr));
    EXPECT(dsa_forward_workspace_size(&b) == 0);
  };
  bad(DSA_ERR_UNSUPPORTED, [](dsa_forward_args& b) { b.mode = 7; });
  bad(DSA_ERR_SHAPE, [](dsa_forward_args& b) { b.T = -1; });
  bad(DSA_ERR_SHAPE, [](dsa_forward_args& b) { b.topk = 0; });
  bad(DSA_ERR_SHAPE, [](dsa_forward_args& b) { b.topk = DSA_MAX_TOPK + 1; });
  bad(DSA_ERR_SHAPE, [](dsa_forward_args& b) { b.q_offset = -1; });
  bad(DSA_ERR_SHAPE, [](dsa_forward_args& b) { b.q_offset = ((int64_t)1 << 31) - 100; });
  bad(DSA_ERR_SHAPE, [](dsa_forward_args& b) { b.flags = DSA_FLAG_DYNAMIC_K; b.dyn_k_min = 4096; });
  bad(DSA_ERR_SHAPE, [](dsa_forward_args& b) { b.flags = DSA_FLAG_DYNAMIC_K; b.dyn_theta = __builtin_nanf(""); });
  bad(DSA_ERR_NULL, [](dsa_forward_args& b) { b.k_idx = nullptr; });
  bad(DSA_ERR_NULL, [](dsa_forward_args& b) { b.k_scale = nullptr; });
  bad(DSA_ERR_NULL, [](dsa_forward_args& b) { b.q_scale = nullptr; });
  bad(DSA_ERR_NULL, [](dsa_forward_args& b) { b.kv = nullptr; });
  bad(DSA_ERR_SHAPE, [](dsa_forward_args& b) { b.k_idx = (const char*)b.k_idx + 16; });
  bad(DSA_ERR_DTYPE, [](dsa_forward_args& b) { b.idx_dtype = DSA_BF16; });
  bad(DSA_ERR_DTYPE, [](dsa_forward_args& b) { b.attn_dtype = DSA_FP8_E4M3; });
  bad(DSA_ERR_UNSUPPORTED, [](dsa_forward_args& b) { b.H = 64; });
  bad(DSA_ERR_UNSUPPORTED, [](dsa_forward_args& b) { b.q_offset = 4000000; });   // rows past 4 GiB of latent KV
  bad(DSA_ERR_SHAPE, [](dsa_forward_args& b) { b.mode = DSA_MODE_DECODE; b.q_offset = 5; b.total_keys = 1000;
                                               b.max_len = 100; b.seq_offsets = (const int64_t*)dptr(13); });
  bad(DSA_ERR_SHAPE, [](dsa_forward_args& b) { b.mode = DSA_MODE_DECODE; b.total_keys = 50; b.max_len = 10;
                                               b.seq_offsets = (const int64_t*)dptr(13); });
  bad(DSA_ERR_SHAPE, [](dsa_forward_args& b) { b.mode = DSA_MODE_DECODE; b.total_keys = 1000; b.max_len = 0;
                                               b.seq_offsets = (const int64_t*)dptr(13); });
  bad(DSA_ERR_NULL, [](dsa_forward_args& b) { b.mode = DSA_MODE_DECODE; b.total_keys = 1000; b.max_len = 10; });
  bad(DSA_ERR_UNSUPPORTED, [](dsa_forward_args& b) { b.mode = DSA_MODE_DECODE; b.total_keys = 1000; b.max_len = 10;
                                                     b.seq_offsets = (const int64_t*)dptr(13); b.idx_dtype = DSA_F32;
                                                     b.q_scale = nullptr; b.k_scale = nullptr; b.w_dtype = DSA_F32; });
}

// dsa_forward_static: the same launches on the library's static scratch,
// which is looked up once per device; above its size nothing is launched
void check_forward_static() {
  int32_t* idx = (int32_t*)dptr(11);
  void* out = dptr(12);
  EXPECT(vars().size() == 1 && vars().begin()->second == DSA_STATIC_SCRATCH_BYTES);
  dsa_forward_args d = prefill_args(64, kAttnShapes[3], true, 2048, 0, 0);
  d.mode = DSA_MODE_DECODE;
  d.seq_offsets = (const int64_t*)dptr(13);
  d.total_keys = (int64_t)64 * 131072;
  d.max_len = 131072;
  const int lookups = g_symbol_lookups;
  CALL(DSA_OK, true, dsa_forward_static(&d, idx, out, nullptr));
  CALL(DSA_OK, true, dsa_forward_static(&d, nullptr, out, nullptr));
  EXPECT(g_symbol_lookups == lookups + 1 || (lookups > 0 && g_symbol_lookups == lookups));
  EXPECT(dsa_forward_workspace_size(&d) <= DSA_STATIC_SCRATCH_BYTES);
  dsa_forward_args p = prefill_args(1000, kAttnShapes[3], true, 256, 0, 0);
  CALL(DSA_OK, true, dsa_forward_static(&p, idx, out, nullptr));
  dsa_forward_args big = prefill_args(6000, kAttnShapes[3], true, 2048, 0, 0);
  EXPECT(dsa_forward_workspace_size(&big) > DSA_STATIC_SCRATCH_BYTES);
  CALL(DSA_ERR_WORKSPACE, false, dsa_forward_static(&big, idx, out, nullptr));
  d.total_keys = (int64_t)64 * 600000;  // scores of every cached key do not fit
  d.max_len = 600000;
  CALL(DSA_ERR_WORKSPACE, false, dsa_forward_static(&d, idx, out, nullptr));
  CALL(DSA_ERR_NULL, false, dsa_forward_static(&p, idx, nullptr, nullptr));
  CALL(DSA_ERR_NULL, false, dsa_forward_static(nullptr, idx, out, nullptr));
  dsa_forward_args e = p;
  e.T = 0;
  CALL(DSA_OK, false, dsa_forward_static(&e, nullptr, nullptr, nullptr));
}

// a device that is not gfx950 is refused before anything is launched
void check_other_device() {
  g_device = 1;
  void *q = dptr(3), *w = dptr(4), *o = dptr(5);
  float *qs = (float*)dptr(6), *os = (float*)dptr(7);
  CALL(DSA_ERR_DEVICE, false, dsa_fold_index_query(q, qs, DSA_FP8_E4M3, w, DSA_BF16, 8, o, os, nullptr));
  {
    dsa_forward_args p = prefill_args(1000, kAttnShapes[3], true, 256, 0, 0);
    CALL(DSA_ERR_DEVICE, false, dsa_forward_static(&p, (int32_t*)dptr(11), dptr(12), nullptr));
  }
  {
    dsa_forward_args a = prefill_args(100, kAttnShapes[3], true, 2048, 0, 0);
    const size_t ws = dsa_forward_workspace_size(&a);
    CALL(DSA_ERR_DEVICE, false, dsa_forward(&a, (int32_t*)dptr(11), dptr(12), kWs, ws, nullptr));
  }
  g_device = 0;
}

}  // namespace

int main() {
  check_misc();
  check_fold();
  check_scores();
  check_topk();
  check_attn();
  check_bwd();
  check_kl();
  check_forward();
  check_forward_static();
  check_other_device();
  std::printf("abi host check: %d checks, %d launches recorded, %d failures\n", g_checks, g_launches, g_failures);
  return g_failures == 0 ? 0 : 1;
}
