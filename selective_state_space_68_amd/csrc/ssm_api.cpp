// C-ABI host layer of libssm.so: argument validation, aliasing checks and
// dispatch to the gfx950 kernels on the caller's stream.  No allocation, no
// synchronisation, no global mutable state beyond a cached device probe.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "../../include/ssm.h"
#include "kernels.hpp"

namespace {

constexpr int kVersion = 30100;  // 3.1.0: + allocation-free SSD entry point (ssm_ssd_scan_fwd_noalloc)

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
  bool empty() const { return lo == hi; }
};

Span span(const void* p, uint64_t bytes) {
  Span s;
  s.lo = reinterpret_cast<uintptr_t>(p);
  s.hi = s.lo + (p ? bytes : 0);
  return s;
}

bool overlaps(const Span& a, const Span& b) {
  if (a.empty() || b.empty()) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) { return !__builtin_mul_overflow(a, b, out); }

bool aligned(const void* p, uintptr_t a) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Bytes of the saved chunk states: [batch][D][ceil(L / 512)][N] float32 (sizes already
// checked by check_scan, so the product does not overflow).
uint64_t chunk_states_bytes(int64_t batch, int64_t L, int64_t D, int64_t N) {
  const uint64_t nck = (static_cast<uint64_t>(L) + ssm::kSaveChunk - 1) / ssm::kSaveChunk;
  return static_cast<uint64_t>(batch) * static_cast<uint64_t>(D) * nck * static_cast<uint64_t>(N) * sizeof(float);
}

// 1 = a device is usable, 0 = none; probed once per process.
std::atomic<int> g_device_state{-1};

ssm_status probe_device() {
  int st = g_device_state.load(std::memory_order_relaxed);
  if (st == 1) return SSM_OK;
  if (st == 0) return SSM_ERR_HIP;
  int count = 0;
  const hipError_t e = hipGetDeviceCount(&count);
  st = (e == hipSuccess && count > 0) ? 1 : 0;
  if (e != hipSuccess) (void)hipGetLastError();
  g_device_state.store(st, std::memory_order_relaxed);
  return st ? SSM_OK : SSM_ERR_HIP;
}

ssm_status from_hip(hipError_t e) { return e == hipSuccess ? SSM_OK : SSM_ERR_HIP; }

struct ScanSizes {
  uint64_t act_bytes = 0, bc_bytes = 0, a_bytes = 0, vec_bytes = 0, state_bytes = 0;
};

ssm_status check_scan(const void* u, const void* delta, const float* A, const void* Bm, const void* Cm,
                      const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                      const float* initial_state, const void* y, const float* final_state, int64_t batch,
                      int64_t L, int64_t D, int64_t N, ssm_dtype dt, ScanSizes* sz) {
  if (dt != SSM_F32 && dt != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (batch < 0 || L < 0 || D < 0 || N < 0) return SSM_ERR_INVALID_ARG;
  if (N < 1 || N > SSM_MAX_N) return SSM_ERR_UNSUPPORTED;
  if (delta_softplus != 0 && delta_softplus != 1) return SSM_ERR_INVALID_ARG;
  const uint64_t e = dt == SSM_BF16 ? 2 : 4;
  uint64_t bd, bdl, bl, bln, dn, bdn;
  if (!mul_ok(batch, D, &bd) || !mul_ok(bd, L, &bdl) || !mul_ok(bdl, e, &sz->act_bytes) ||
      !mul_ok(batch, L, &bl) || !mul_ok(bl, N, &bln) || !mul_ok(bln, e, &sz->bc_bytes) ||
      !mul_ok(D, N, &dn) || !mul_ok(dn, 4, &sz->a_bytes) || !mul_ok(bd, N, &bdn) ||
      !mul_ok(bdn, 4, &sz->state_bytes) || sz->act_bytes > (uint64_t(1) << 62))
    return SSM_ERR_INVALID_ARG;
  // Required pointers may be NULL only when the buffer they describe is empty.
  if ((!u && sz->act_bytes) || (!delta && sz->act_bytes) || (!y && sz->act_bytes) ||
      (!Bm && sz->bc_bytes) || (!Cm && sz->bc_bytes) || (!A && sz->a_bytes))
    return SSM_ERR_INVALID_ARG;
  sz->vec_bytes = static_cast<uint64_t>(D) * 4;
  if (!aligned(u, e) || !aligned(delta, e) || !aligned(z, e) || !aligned(y, e) || !aligned(Bm, e) ||
      !aligned(Cm, e) || !aligned(A, 4) || !aligned(Dskip, 4) || !aligned(delta_bias, 4) ||
      !aligned(final_state, 4) || !aligned(initial_state, 4))
    return SSM_ERR_INVALID_ARG;
  const Span in[] = {span(u, sz->act_bytes),        span(delta, sz->act_bytes),
                     span(z, sz->act_bytes),        span(A, sz->a_bytes),
                     span(Bm, sz->bc_bytes),        span(Cm, sz->bc_bytes),
                     span(Dskip, sz->vec_bytes),    span(delta_bias, sz->vec_bytes)};
  const Span ys = span(y, sz->act_bytes);
  const Span fs = span(final_state, sz->state_bytes);
  const Span hs = span(initial_state, sz->state_bytes);
  for (const Span& s : in)
    if (overlaps(ys, s) || overlaps(fs, s) || overlaps(hs, s)) return SSM_ERR_INVALID_ARG;
  if (overlaps(ys, fs) || overlaps(ys, hs)) return SSM_ERR_INVALID_ARG;
  // the final state may replace the initial state in place, but not partly overlap it
  if (overlaps(hs, fs) && initial_state != final_state) return SSM_ERR_INVALID_ARG;
  return SSM_OK;
}

}  // namespace

namespace ssm {

ssm_status ssd_check(const void* x, const void* dt, const float* A, const void* Bm, const void* Cm, const float* Dskip,
                     const float* dt_bias, int dt_softplus, const float* initial_state, const void* y,
                     const float* final_state, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                     ssm_dtype dtype, const void* workspace, size_t workspace_bytes, SsdArgs* a) {
  if (dtype != SSM_F32 && dtype != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (batch < 0 || L < 0 || H < 0 || P < 0 || N < 0) return SSM_ERR_INVALID_ARG;
  if (dt_softplus != 0 && dt_softplus != 1) return SSM_ERR_INVALID_ARG;
  if (dtype != SSM_BF16 || !ssd_supported(H, P, N)) return SSM_ERR_UNSUPPORTED;
  uint64_t blh, xe, xbytes, dtbytes, bl, bcbytes, bh, st, stbytes;
  if (!mul_ok(batch, L, &blh) || !mul_ok(blh, H, &blh) || !mul_ok(blh, P, &xe) || !mul_ok(xe, 2, &xbytes) ||
      !mul_ok(batch, L, &bl) || !mul_ok(bl, H, &dtbytes) || !mul_ok(dtbytes, 2, &dtbytes) ||
      !mul_ok(bl, N, &bcbytes) || !mul_ok(bcbytes, 2, &bcbytes) || !mul_ok(batch, H, &bh) ||
      !mul_ok(bh, P * N, &st) || !mul_ok(st, 4, &stbytes) || xbytes > (uint64_t(1) << 62))
    return SSM_ERR_INVALID_ARG;
  const uint64_t hbytes = static_cast<uint64_t>(H) * 4;
  if ((!x && xbytes) || (!y && xbytes) || (!dt && dtbytes) || (!Bm && bcbytes) || (!Cm && bcbytes) ||
      (!A && hbytes))
    return SSM_ERR_INVALID_ARG;
  // the kernel moves 16-byte vectors of x, y, B, C and the states
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(Bm, 16) || !aligned(Cm, 16) || !aligned(dt, 2) ||
      !aligned(A, 4) || !aligned(Dskip, 4) || !aligned(dt_bias, 4) || !aligned(initial_state, 16) ||
      !aligned(final_state, 16) || !aligned(workspace, 16))
    return SSM_ERR_INVALID_ARG;
  if (workspace_bytes && !workspace) return SSM_ERR_INVALID_ARG;
  const Span ys = span(y, xbytes), fs = span(final_state, stbytes), hs = span(initial_state, stbytes);
  const Span in[] = {span(x, xbytes),       span(dt, dtbytes),     span(A, hbytes),    span(Bm, bcbytes),
                     span(Cm, bcbytes),     span(Dskip, hbytes),   span(dt_bias, hbytes)};
  for (const Span& s : in)
    if (overlaps(ys, s) || overlaps(fs, s) || overlaps(hs, s)) return SSM_ERR_INVALID_ARG;
  if (overlaps(ys, fs) || overlaps(ys, hs)) return SSM_ERR_INVALID_ARG;
  // the final state may replace the initial state in place, but not partly overlap it
  if (overlaps(hs, fs) && initial_state != final_state) return SSM_ERR_INVALID_ARG;
  const Span wsp = span(workspace, workspace_bytes);
  for (const Span& s : in)
    if (overlaps(wsp, s)) return SSM_ERR_INVALID_ARG;
  if (overlaps(wsp, ys) || overlaps(wsp, fs) || overlaps(wsp, hs)) return SSM_ERR_INVALID_ARG;
  a->x = x; a->dt = dt; a->A = A; a->Bm = Bm; a->Cm = Cm; a->Dskip = Dskip; a->dt_bias = dt_bias;
  a->h0 = initial_state; a->y = const_cast<void*>(y); a->final_state = const_cast<float*>(final_state);
  a->batch = batch; a->L = L; a->H = H; a->P = static_cast<int>(P); a->N = static_cast<int>(N);
  a->softplus = dt_softplus;
  return SSM_OK;
}

ssm_status ssd_run(const SsdArgs& a, void* workspace, size_t workspace_bytes, void* stream) {
  if (a.batch == 0 || a.H == 0) return SSM_OK;
  const ssm_status ds = probe_device();
  if (ds != SSM_OK) return ds;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.L == 0)
    return a.final_state
               ? from_hip(launch_copy_state(a.final_state, a.h0, a.batch * a.H * a.P * a.N, s))
               : SSM_OK;
  return from_hip(launch_ssd_scan(a, workspace, workspace_bytes, s));
}

}  // namespace ssm

extern "C" {

size_t ssm_ssd_scan_workspace_size(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, ssm_dtype dtype) {
  if (dtype != SSM_BF16 || !ssm::ssd_supported(H, P, N) || batch <= 0 || L <= 0 || H <= 0) return 0;
  uint64_t t;
  if (!mul_ok(batch, H, &t) || !mul_ok(t, L, &t) || t > (uint64_t(1) << 50)) return 0;
  return ssm::ssd_workspace_bytes(batch, L, H, P, N);
}

ssm_status ssm_ssd_scan_fwd(const void* x, const void* dt, const float* A, const void* Bm, const void* Cm,
                            const float* Dskip, const float* dt_bias, int dt_softplus, const float* initial_state,
                            void* y, float* final_state, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                            ssm_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  ssm::SsdArgs a;
  const ssm_status st = ssm::ssd_check(x, dt, A, Bm, Cm, Dskip, dt_bias, dt_softplus, initial_state, y, final_state,
                                       batch, L, H, P, N, dtype, workspace, workspace_bytes, &a);
  if (st != SSM_OK) return st;
  return ssm::ssd_run(a, workspace, workspace_bytes, stream);
}

const char* ssm_status_string(ssm_status s) {
  switch (s) {
    case SSM_OK: return "SSM_OK: success";
    case SSM_ERR_INVALID_ARG: return "SSM_ERR_INVALID_ARG: invalid argument (null pointer, negative size, misalignment or aliasing)";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED: unsupported configuration (N outside [1, 64], dtype or variant)";
    case SSM_ERR_HIP: return "SSM_ERR_HIP: HIP runtime error (no usable device, or launch failed)";
    case SSM_ERR_TOO_LARGE:
      return "SSM_ERR_TOO_LARGE: the call needs more scratch than the allocation-free entry point holds";
  }
  return "SSM: unknown status";
}

int ssm_version(void) { return kVersion; }

}  // extern "C"

namespace {

// The per-kernel option: tokens per lane of the chunked kernel (8 or 16), states
// per lane of the token-sequential kernel (2 or 4); 0 = default.
bool kernel_option_ok(int variant, int tokens_per_lane) {
  if (variant == SSM_SCAN_TOKSEQ) return tokens_per_lane == 0 || tokens_per_lane == 2 || tokens_per_lane == 4;
  return tokens_per_lane == 0 || tokens_per_lane == 8 || tokens_per_lane == 12 || tokens_per_lane == 16;
}

// The kernel a scan with these arguments runs (L > 0): SSM_SCAN_SEQUENTIAL,
// SSM_SCAN_CHUNKED or SSM_SCAN_TOKSEQ, or minus SSM_ERR_UNSUPPORTED.
int choose_scan_kernel(const ssm::ScanArgs& a, ssm::Dt d, int variant, int tokens_per_lane) {
  const bool tokseq = (variant == SSM_SCAN_TOKSEQ && ssm::tokseq_supported(a)) ||
                      (variant == SSM_SCAN_AUTO && tokens_per_lane == 0 && ssm::tokseq_preferred(a, d));
  if (variant == SSM_SCAN_TOKSEQ && !tokseq) return -SSM_ERR_UNSUPPORTED;
  if (tokseq) return SSM_SCAN_TOKSEQ;
  const bool chunked = (variant == SSM_SCAN_AUTO || variant == SSM_SCAN_CHUNKED) &&
                       ssm::chunked_supported(a, d, tokens_per_lane);
  if (variant == SSM_SCAN_CHUNKED && !chunked) return -SSM_ERR_UNSUPPORTED;
  // the sequential kernel has neither the full hold nor the fused conv
  if ((a.zoh || a.conv_w != nullptr) && !chunked) return -SSM_ERR_UNSUPPORTED;
  return chunked ? SSM_SCAN_CHUNKED : SSM_SCAN_SEQUENTIAL;
}

// The caller's workspace for a forward scan: NULL with a zero size, or a 16-byte
// aligned buffer of at least `need` bytes that overlaps no other argument.
ssm_status check_scan_workspace(const void* workspace, size_t workspace_bytes, size_t need, const void* u,
                                const void* delta, const float* A, const void* Bm, const void* Cm, const float* Dskip,
                                const void* z, const float* delta_bias, const float* initial_state, const void* y,
                                const float* final_state, const ScanSizes& sz) {
  if (workspace_bytes && !workspace) return SSM_ERR_INVALID_ARG;
  if (workspace_bytes < need || !aligned(workspace, 16)) return SSM_ERR_INVALID_ARG;
  const Span ws = span(workspace, workspace_bytes);
  const Span all[] = {span(u, sz.act_bytes),           span(delta, sz.act_bytes),     span(z, sz.act_bytes),
                      span(A, sz.a_bytes),             span(Bm, sz.bc_bytes),         span(Cm, sz.bc_bytes),
                      span(Dskip, sz.vec_bytes),       span(delta_bias, sz.vec_bytes),
                      span(initial_state, sz.state_bytes), span(y, sz.act_bytes),
                      span(final_state, sz.state_bytes)};
  for (const Span& o : all)
    if (overlaps(ws, o)) return SSM_ERR_INVALID_ARG;
  return SSM_OK;
}

// Workspace bytes a forward scan of this shape uses: none.  The kernels need no
// device memory beyond their arguments; a wave walks all of L for its channel, so
// no carry crosses workgroups through memory.
size_t scan_workspace_need(int64_t, int64_t, int64_t, int64_t, ssm_dtype) { return 0; }

ssm_status scan_fwd(const void* u, const void* delta, const float* A, const void* Bm, const void* Cm,
                    const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                    const float* initial_state, void* y, float* final_state, int64_t batch, int64_t L, int64_t D,
                    int64_t N, ssm_dtype dt, void* workspace, size_t workspace_bytes, void* stream, int variant,
                    int tokens_per_lane, int zoh, float* chunk_states = nullptr) {
  ScanSizes sz;
  ssm_status st = check_scan(u, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, initial_state, y,
                             final_state, batch, L, D, N, dt, &sz);
  if (st != SSM_OK) return st;
  st = check_scan_workspace(workspace, workspace_bytes, scan_workspace_need(batch, L, D, N, dt), u, delta, A, Bm, Cm,
                            Dskip, z, delta_bias, initial_state, y, final_state, sz);
  if (st != SSM_OK) return st;
  if (chunk_states) {
    if (N > 16) return SSM_ERR_UNSUPPORTED;
    if (!aligned(chunk_states, 16)) return SSM_ERR_INVALID_ARG;
    const uint64_t cs_bytes = chunk_states_bytes(batch, L, D, N);
    const Span cs = span(chunk_states, cs_bytes);
    const Span all[] = {span(u, sz.act_bytes),           span(delta, sz.act_bytes),     span(z, sz.act_bytes),
                        span(A, sz.a_bytes),             span(Bm, sz.bc_bytes),         span(Cm, sz.bc_bytes),
                        span(Dskip, sz.vec_bytes),       span(delta_bias, sz.vec_bytes),
                        span(initial_state, sz.state_bytes), span(y, sz.act_bytes),
                        span(final_state, sz.state_bytes), span(workspace, workspace_bytes)};
    for (const Span& o : all)
      if (overlaps(cs, o)) return SSM_ERR_INVALID_ARG;
  }
  const int ap = (variant & SSM_SCAN_AP) ? 1 : 0;
  variant &= ~SSM_SCAN_AP;
  if (variant != SSM_SCAN_AUTO && variant != SSM_SCAN_SEQUENTIAL && variant != SSM_SCAN_CHUNKED &&
      variant != SSM_SCAN_TOKSEQ)
    return SSM_ERR_UNSUPPORTED;
  if (!kernel_option_ok(variant, tokens_per_lane)) return SSM_ERR_UNSUPPORTED;
  if (batch == 0 || D == 0) return SSM_OK;  // nothing to compute or write
  ssm::ScanArgs a;
  a.u = u; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip; a.z = z;
  a.bias = delta_bias; a.h0 = initial_state; a.y = y; a.final_state = final_state;
  a.batch = batch; a.L = L; a.D = D; a.N = static_cast<int>(N); a.softplus = delta_softplus; a.zoh = zoh;
  a.ap = ap;
  a.chunk_states = chunk_states;
  const ssm::Dt d = dt == SSM_BF16 ? ssm::Dt::BF16 : ssm::Dt::F32;
  const int kernel = L > 0 ? choose_scan_kernel(a, d, variant, tokens_per_lane) : SSM_SCAN_SEQUENTIAL;
  // the saved states are 512-token chunks: the chunked kernel runs at 8 tokens per lane
  if (chunk_states) tokens_per_lane = 8;
  if (kernel < 0) return static_cast<ssm_status>(-kernel);
  const bool tokseq = L > 0 && kernel == SSM_SCAN_TOKSEQ;
  // saving the chunk states: the chunked kernel's saving build covers N == 16 on the
  // vector path; other shapes save through the sequential kernel
  const bool chunked = L > 0 && kernel == SSM_SCAN_CHUNKED && (!chunk_states || ssm::chunked_save_supported(a));
  st = probe_device();
  if (st != SSM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L == 0)  // the final state is the initial state
    return final_state ? from_hip(ssm::launch_copy_state(final_state, initial_state, batch * D * N, s)) : SSM_OK;
  if (tokseq) return from_hip(ssm::launch_scan_tokseq(a, d, chunk_states ? 0 : tokens_per_lane, s));
  if (chunked) return from_hip(ssm::launch_scan_chunked(a, d, tokens_per_lane, s));
  return from_hip(ssm::launch_scan_sequential(a, d, s));
}

}  // namespace

extern "C" {

size_t ssm_selective_scan_workspace_size(int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt) {
  if (dt != SSM_F32 && dt != SSM_BF16) return 0;
  if (batch <= 0 || L <= 0 || D <= 0 || N < 1 || N > SSM_MAX_N) return 0;
  return scan_workspace_need(batch, L, D, N, dt);
}

ssm_status ssm_selective_scan_fwd_variant(const void* u, const void* delta, const float* A, const void* Bm,
                                          const void* Cm, const float* Dskip, const void* z,
                                          const float* delta_bias, int delta_softplus,
                                          const float* initial_state, void* y, float* final_state,
                                          int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
                                          void* workspace, size_t workspace_bytes, void* stream, int variant,
                                          int tokens_per_lane) {
  return scan_fwd(u, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, initial_state, y, final_state, batch, L,
                  D, N, dt, workspace, workspace_bytes, stream, variant, tokens_per_lane, 0);
}

int ssm_selective_scan_fwd_kernel(int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt, int gate, int zoh,
                                  int conv_width, int variant, int tokens_per_lane) {
  if (dt != SSM_F32 && dt != SSM_BF16) return -SSM_ERR_UNSUPPORTED;
  if (batch <= 0 || L <= 0 || D <= 0 || N < 1) return -SSM_ERR_INVALID_ARG;
  if (N > SSM_MAX_N) return -SSM_ERR_UNSUPPORTED;
  variant &= ~SSM_SCAN_AP;                           // (the decay path does not change the kernel)
  if (variant != SSM_SCAN_AUTO && variant != SSM_SCAN_SEQUENTIAL && variant != SSM_SCAN_CHUNKED &&
      variant != SSM_SCAN_TOKSEQ)
    return -SSM_ERR_UNSUPPORTED;
  if (!kernel_option_ok(variant, tokens_per_lane)) return -SSM_ERR_UNSUPPORTED;
  if (conv_width < 0 || conv_width > SSM_MAX_CONV_WIDTH || (zoh && conv_width)) return -SSM_ERR_UNSUPPORTED;
  if ((zoh || conv_width) && variant != SSM_SCAN_AUTO) return -SSM_ERR_UNSUPPORTED;   // (those entry points choose)
  // stand-in pointers: 256-byte aligned, never dereferenced
  void* const any = reinterpret_cast<void*>(uintptr_t(256));
  ssm::ScanArgs a;
  a.u = any; a.delta = any; a.A = static_cast<const float*>(any); a.Bm = any; a.Cm = any; a.Dskip = nullptr;
  a.z = gate ? any : nullptr; a.bias = nullptr; a.h0 = nullptr; a.y = any; a.final_state = nullptr;
  a.batch = batch; a.L = L; a.D = D; a.N = static_cast<int>(N); a.softplus = 1; a.zoh = zoh ? 1 : 0;
  if (conv_width) { a.conv_w = static_cast<const float*>(any); a.conv_k = conv_width; }
  return choose_scan_kernel(a, dt == SSM_BF16 ? ssm::Dt::BF16 : ssm::Dt::F32, variant, tokens_per_lane);
}

ssm_status ssm_selective_scan_fwd_zoh(const void* u, const void* delta, const float* A, const void* Bm,
                                      const void* Cm, const float* Dskip, const void* z, const float* delta_bias,
                                      int delta_softplus, const float* initial_state, void* y, float* final_state,
                                      int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt, void* stream) {
  return scan_fwd(u, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, initial_state, y, final_state, batch, L,
                  D, N, dt, nullptr, 0, stream, SSM_SCAN_AUTO, 0, 1);
}

ssm_status ssm_selective_scan_fwd(const void* u, const void* delta, const float* A, const void* Bm,
                                  const void* Cm, const float* Dskip, const void* z, const float* delta_bias,
                                  int delta_softplus, void* y, float* final_state, int64_t batch, int64_t L,
                                  int64_t D, int64_t N, ssm_dtype dt, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return scan_fwd(u, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, nullptr, y, final_state, batch, L, D, N,
                  dt, workspace, workspace_bytes, stream, SSM_SCAN_AUTO, 0, 0);
}

ssm_status ssm_selective_scan_fwd_from_state(const void* u, const void* delta, const float* A, const void* Bm,
                                             const void* Cm, const float* Dskip, const void* z,
                                             const float* delta_bias, int delta_softplus,
                                             const float* initial_state, void* y, float* final_state,
                                             int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
                                             void* workspace, size_t workspace_bytes, void* stream) {
  return scan_fwd(u, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, initial_state, y, final_state, batch, L,
                  D, N, dt, workspace, workspace_bytes, stream, SSM_SCAN_AUTO, 0, 0);
}

ssm_status ssm_selective_scan_fwd_save(const void* u, const void* delta, const float* A, const void* Bm,
                                       const void* Cm, const float* Dskip, const void* z, const float* delta_bias,
                                       int delta_softplus, const float* initial_state, void* y, float* final_state,
                                       float* chunk_states, int64_t batch, int64_t L, int64_t D, int64_t N,
                                       ssm_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
  if (!chunk_states && batch > 0 && L > 0 && D > 0 && N > 0) return SSM_ERR_INVALID_ARG;
  return scan_fwd(u, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, initial_state, y, final_state, batch, L,
                  D, N, dt, workspace, workspace_bytes, stream, SSM_SCAN_AUTO, 0, 0, chunk_states);
}

ssm_status ssm_selective_scan_fwd_conv(const void* x, const float* conv_w, const float* conv_b, int64_t conv_width,
                                       const void* delta, const float* A, const void* Bm, const void* Cm,
                                       const float* Dskip, const void* z, const float* delta_bias,
                                       int delta_softplus, const float* initial_state, void* u_out, void* y,
                                       float* final_state, int64_t batch, int64_t L, int64_t D, int64_t N,
                                       ssm_dtype dt, void* stream, int tokens_per_lane) {
  ScanSizes sz;
  ssm_status st = check_scan(x, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, initial_state, y,
                             final_state, batch, L, D, N, dt, &sz);
  if (st != SSM_OK) return st;
  if (conv_width < 1 || conv_width > SSM_MAX_CONV_WIDTH) return SSM_ERR_UNSUPPORTED;
  if (!(tokens_per_lane == 0 || tokens_per_lane == 8 || tokens_per_lane == 16)) return SSM_ERR_UNSUPPORTED;
  uint64_t wbytes = 0;
  if (!mul_ok(D, conv_width, &wbytes) || !mul_ok(wbytes, 4, &wbytes)) return SSM_ERR_INVALID_ARG;
  if ((!conv_w && wbytes) || !aligned(conv_w, 4) || !aligned(conv_b, 4) || !aligned(u_out, dt == SSM_BF16 ? 2 : 4))
    return SSM_ERR_INVALID_ARG;
  // u_out is an output: it must not overlap any input or the other outputs
  const Span uo = span(u_out, sz.act_bytes);
  const Span others[] = {span(x, sz.act_bytes),          span(delta, sz.act_bytes),   span(z, sz.act_bytes),
                         span(A, sz.a_bytes),            span(Bm, sz.bc_bytes),       span(Cm, sz.bc_bytes),
                         span(Dskip, sz.vec_bytes),      span(delta_bias, sz.vec_bytes),
                         span(initial_state, sz.state_bytes), span(y, sz.act_bytes),
                         span(final_state, sz.state_bytes), span(conv_w, wbytes),     span(conv_b, sz.vec_bytes)};
  for (const Span& o : others)
    if (overlaps(uo, o)) return SSM_ERR_INVALID_ARG;
  const Span ws = span(conv_w, wbytes), bs = span(conv_b, sz.vec_bytes);
  if (overlaps(ws, span(y, sz.act_bytes)) || overlaps(ws, span(final_state, sz.state_bytes)) ||
      overlaps(bs, span(y, sz.act_bytes)) || overlaps(bs, span(final_state, sz.state_bytes)))
    return SSM_ERR_INVALID_ARG;
  if (batch == 0 || D == 0) return SSM_OK;
  st = probe_device();
  if (st != SSM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L == 0)
    return final_state ? from_hip(ssm::launch_copy_state(final_state, initial_state, batch * D * N, s)) : SSM_OK;
  ssm::ScanArgs a;
  a.u = x; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip; a.z = z;
  a.bias = delta_bias; a.h0 = initial_state; a.y = y; a.final_state = final_state;
  a.batch = batch; a.L = L; a.D = D; a.N = static_cast<int>(N); a.softplus = delta_softplus;
  a.conv_w = conv_w; a.conv_b = conv_b; a.conv_k = static_cast<int>(conv_width); a.u_out = u_out;
  const ssm::Dt d = dt == SSM_BF16 ? ssm::Dt::BF16 : ssm::Dt::F32;
  const int kernel = choose_scan_kernel(a, d, SSM_SCAN_AUTO, tokens_per_lane);
  if (kernel < 0) return static_cast<ssm_status>(-kernel);
  if (kernel == SSM_SCAN_TOKSEQ) return from_hip(ssm::launch_scan_tokseq(a, d, 0, s));
  return from_hip(ssm::launch_scan_chunked(a, d, tokens_per_lane, s));
}

ssm_status ssm_causal_conv1d_fwd(const void* x, const float* conv_w, const float* conv_b, int64_t conv_width,
                                 int apply_silu, void* out, int64_t batch, int64_t D, int64_t L, ssm_dtype dt,
                                 void* stream) {
  if (dt != SSM_F32 && dt != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (batch < 0 || D < 0 || L < 0) return SSM_ERR_INVALID_ARG;
  if (conv_width < 1 || conv_width > SSM_MAX_CONV_WIDTH) return SSM_ERR_UNSUPPORTED;
  if (apply_silu != 0 && apply_silu != 1) return SSM_ERR_INVALID_ARG;
  const uint64_t e = dt == SSM_BF16 ? 2 : 4;
  uint64_t bd, bdl, xbytes, wbytes;
  if (!mul_ok(batch, D, &bd) || !mul_ok(bd, L, &bdl) || !mul_ok(bdl, e, &xbytes) ||
      !mul_ok(D, conv_width, &wbytes) || !mul_ok(wbytes, 4, &wbytes) || xbytes > (uint64_t(1) << 62))
    return SSM_ERR_INVALID_ARG;
  if ((!x && xbytes) || (!out && xbytes) || (!conv_w && wbytes)) return SSM_ERR_INVALID_ARG;
  if (!aligned(x, e) || !aligned(out, e) || !aligned(conv_w, 4) || !aligned(conv_b, 4)) return SSM_ERR_INVALID_ARG;
  const Span os = span(out, xbytes);
  if (overlaps(os, span(x, xbytes)) || overlaps(os, span(conv_w, wbytes)) ||
      overlaps(os, span(conv_b, static_cast<uint64_t>(D) * 4)))
    return SSM_ERR_INVALID_ARG;
  if (xbytes == 0) return SSM_OK;
  const ssm_status st = probe_device();
  if (st != SSM_OK) return st;
  ssm::ConvArgs a;
  a.x = x; a.w = conv_w; a.bias = conv_b; a.out = out;
  a.batch = batch; a.D = D; a.L = L; a.K = static_cast<int>(conv_width); a.silu = apply_silu;
  return from_hip(ssm::launch_causal_conv1d(a, dt == SSM_BF16 ? ssm::Dt::BF16 : ssm::Dt::F32,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

size_t bwd_workspace(int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt, bool saved) {
  if (dt != SSM_F32 && dt != SSM_BF16) return 0;
  if (batch <= 0 || L <= 0 || D <= 0 || N < 1 || N > SSM_MAX_N) return 0;
  uint64_t t;
  if (!mul_ok(batch, D, &t) || !mul_ok(t, L, &t) || t > (uint64_t(1) << 58)) return 0;
  return ssm::scan_bwd_workspace_bytes(batch, L, D, static_cast<int>(N), saved);
}

// chunk_states: null for the plain backward pass, else the forward pass's saved
// chunk states (used where the shape suits the chunk walk, ignored otherwise).
ssm_status scan_bwd(const void* u, const void* delta, const float* A, const void* Bm, const void* Cm,
                    const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                    const float* initial_state, const void* dy, const float* dfinal_state, const float* chunk_states,
                    void* du, void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
                    float* dinitial_state, int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const bool saved = chunk_states != nullptr;
  ScanSizes sz;
  // the forward checks cover the inputs (du stands in for y: required, act-sized)
  ssm_status st = check_scan(u, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, initial_state, du,
                             nullptr, batch, L, D, N, dt, &sz);
  if (st != SSM_OK) return st;
  const uint64_t e = dt == SSM_BF16 ? 2 : 4;
  if ((!dy && sz.act_bytes) || (!ddelta && sz.act_bytes) || (!dB && sz.bc_bytes) || (!dC && sz.bc_bytes) ||
      (!dA && sz.a_bytes))
    return SSM_ERR_INVALID_ARG;
  if (dz && !z) return SSM_ERR_INVALID_ARG;  // no gate: there is no z to differentiate
  if (!aligned(dy, e) || !aligned(ddelta, e) || !aligned(dB, e) || !aligned(dC, e) || !aligned(dz, e) ||
      !aligned(dA, 4) || !aligned(dD, 4) || !aligned(ddelta_bias, 4) || !aligned(dinitial_state, 4) ||
      !aligned(dfinal_state, 4) || !aligned(chunk_states, 4) || !aligned(workspace, 16))
    return SSM_ERR_INVALID_ARG;
  const uint64_t cs_bytes = saved ? chunk_states_bytes(batch, L, D, N) : 0;
  const Span ins[] = {span(u, sz.act_bytes),         span(delta, sz.act_bytes),      span(z, sz.act_bytes),
                      span(A, sz.a_bytes),           span(Bm, sz.bc_bytes),          span(Cm, sz.bc_bytes),
                      span(Dskip, sz.vec_bytes),     span(delta_bias, sz.vec_bytes), span(initial_state, sz.state_bytes),
                      span(dy, sz.act_bytes),        span(dfinal_state, sz.state_bytes), span(chunk_states, cs_bytes)};
  const size_t need = bwd_workspace(batch, L, D, N, dt, saved);
  const Span outs[] = {span(du, sz.act_bytes),          span(ddelta, sz.act_bytes),   span(dA, sz.a_bytes),
                       span(dB, sz.bc_bytes),           span(dC, sz.bc_bytes),        span(dD, sz.vec_bytes),
                       span(dz, sz.act_bytes),          span(ddelta_bias, sz.vec_bytes),
                       span(dinitial_state, sz.state_bytes), span(workspace, need)};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const Span& s : ins)
      if (overlaps(outs[i], s)) return SSM_ERR_INVALID_ARG;
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlaps(outs[i], outs[j])) return SSM_ERR_INVALID_ARG;
  }
  if (workspace_bytes < need || (need && !workspace)) return SSM_ERR_INVALID_ARG;
  if (!ssm::scan_bwd_grid_ok(batch, L, D, static_cast<int>(N))) return SSM_ERR_UNSUPPORTED;
  if (D == 0) return SSM_OK;  // every output is empty
  st = probe_device();
  if (st != SSM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (batch == 0 || L == 0) {
    // sums over no tokens are zero; with no tokens the final state is the initial
    // state, so its cotangent passes straight to the initial state
    hipError_t he = ssm::launch_copy_state(dA, nullptr, D * N, s);
    if (he == hipSuccess && dD) he = ssm::launch_copy_state(dD, nullptr, D, s);
    if (he == hipSuccess && ddelta_bias) he = ssm::launch_copy_state(ddelta_bias, nullptr, D, s);
    if (he == hipSuccess && dinitial_state)
      he = ssm::launch_copy_state(dinitial_state, dfinal_state, batch * D * N, s);
    return from_hip(he);
  }
  ssm::BwdArgs a;
  a.u = u; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dskip = Dskip; a.z = z; a.bias = delta_bias;
  a.h0 = initial_state; a.dy = dy; a.dfinal = dfinal_state; a.chunk_states = chunk_states;
  a.du = du; a.ddelta = ddelta; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD; a.dz = dz; a.dbias = ddelta_bias;
  a.dh0 = dinitial_state;
  a.batch = batch; a.L = L; a.D = D; a.N = static_cast<int>(N); a.softplus = delta_softplus;
  return from_hip(ssm::launch_scan_bwd(a, dt == SSM_BF16 ? ssm::Dt::BF16 : ssm::Dt::F32, workspace, s));
}

}  // namespace

extern "C" {

size_t ssm_selective_scan_bwd_workspace_size(int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt) {
  return bwd_workspace(batch, L, D, N, dt, false);
}

size_t ssm_selective_scan_bwd_saved_workspace_size(int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt) {
  return bwd_workspace(batch, L, D, N, dt, true);
}

ssm_status ssm_selective_scan_bwd(const void* u, const void* delta, const float* A, const void* Bm, const void* Cm,
                                  const float* Dskip, const void* z, const float* delta_bias, int delta_softplus,
                                  const float* initial_state, const void* dy, const float* dfinal_state, void* du,
                                  void* ddelta, float* dA, void* dB, void* dC, float* dD, void* dz,
                                  float* ddelta_bias, float* dinitial_state, int64_t batch, int64_t L, int64_t D,
                                  int64_t N, ssm_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
  return scan_bwd(u, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, initial_state, dy, dfinal_state, nullptr,
                  du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state, batch, L, D, N, dt, workspace,
                  workspace_bytes, stream);
}

ssm_status ssm_selective_scan_bwd_saved(const void* u, const void* delta, const float* A, const void* Bm,
                                        const void* Cm, const float* Dskip, const void* z, const float* delta_bias,
                                        int delta_softplus, const float* initial_state, const void* dy,
                                        const float* dfinal_state, const float* chunk_states, void* du, void* ddelta,
                                        float* dA, void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
                                        float* dinitial_state, int64_t batch, int64_t L, int64_t D, int64_t N,
                                        ssm_dtype dt, void* workspace, size_t workspace_bytes, void* stream) {
  if (!chunk_states && batch > 0 && L > 0 && D > 0 && N > 0) return SSM_ERR_INVALID_ARG;
  return scan_bwd(u, delta, A, Bm, Cm, Dskip, z, delta_bias, delta_softplus, initial_state, dy, dfinal_state,
                  chunk_states, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dinitial_state,
                  batch, L, D, N, dt, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

ssm_status state_update(const float* state_in, float* state_out, const void* u_t, const void* delta_t,
                        const float* A, const void* B_t, const void* C_t, const float* Dskip, const void* z_t,
                        const float* delta_bias, int delta_softplus, void* y_t, int64_t batch, int64_t D, int64_t N,
                        ssm_dtype dt, void* stream, int zoh) {
  if (dt != SSM_F32 && dt != SSM_BF16) return SSM_ERR_UNSUPPORTED;
  if (batch < 0 || D < 0 || N < 0) return SSM_ERR_INVALID_ARG;
  if (N < 1 || N > SSM_MAX_N) return SSM_ERR_UNSUPPORTED;
  if (delta_softplus != 0 && delta_softplus != 1) return SSM_ERR_INVALID_ARG;
  const uint64_t e = dt == SSM_BF16 ? 2 : 4;
  uint64_t bd, bdn, st_bytes, act_bytes, bn, bc_bytes, dn;
  if (!mul_ok(batch, D, &bd) || !mul_ok(bd, N, &bdn) || !mul_ok(bdn, 4, &st_bytes) ||
      !mul_ok(bd, e, &act_bytes) || !mul_ok(batch, N, &bn) || !mul_ok(bn, e, &bc_bytes) ||
      !mul_ok(D, N, &dn) || st_bytes > (uint64_t(1) << 62))
    return SSM_ERR_INVALID_ARG;
  // Required pointers may be NULL only when the buffer they describe is empty.
  if ((!state_in && st_bytes) || (!state_out && st_bytes) || (!u_t && act_bytes) || (!delta_t && act_bytes) ||
      (!y_t && act_bytes) || (!B_t && bc_bytes) || (!C_t && bc_bytes) || (!A && dn))
    return SSM_ERR_INVALID_ARG;
  if (!aligned(state_in, 4) || !aligned(state_out, 4) || !aligned(A, 4) || !aligned(Dskip, 4) ||
      !aligned(delta_bias, 4) || !aligned(u_t, e) || !aligned(delta_t, e) || !aligned(z_t, e) ||
      !aligned(B_t, e) || !aligned(C_t, e) || !aligned(y_t, e))
    return SSM_ERR_INVALID_ARG;
  const Span sin = span(state_in, st_bytes), sout = span(state_out, st_bytes), ys = span(y_t, act_bytes);
  const Span in[] = {span(u_t, act_bytes),         span(delta_t, act_bytes),    span(z_t, act_bytes),
                     span(A, dn * 4),              span(B_t, bc_bytes),         span(C_t, bc_bytes),
                     span(Dskip, uint64_t(D) * 4), span(delta_bias, uint64_t(D) * 4)};
  for (const Span& s : in)
    if (overlaps(ys, s) || overlaps(sout, s)) return SSM_ERR_INVALID_ARG;
  if (overlaps(ys, sin) || overlaps(ys, sout)) return SSM_ERR_INVALID_ARG;
  if (sin.lo != sout.lo && overlaps(sin, sout)) return SSM_ERR_INVALID_ARG;  // exact in-place only
  if (batch == 0 || D == 0) return SSM_OK;  // nothing to compute or write
  const ssm_status dst = probe_device();
  if (dst != SSM_OK) return dst;

  ssm::StepArgs a;
  a.state_in = state_in; a.state_out = state_out; a.u = u_t; a.delta = delta_t; a.A = A; a.Bm = B_t;
  a.Cm = C_t; a.Dskip = Dskip; a.z = z_t; a.bias = delta_bias; a.y = y_t;
  a.batch = batch; a.D = D; a.N = static_cast<int>(N); a.softplus = delta_softplus; a.zoh = zoh;
  return from_hip(ssm::launch_state_update(a, dt == SSM_BF16 ? ssm::Dt::BF16 : ssm::Dt::F32,
                                           static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

ssm_status ssm_state_update(const float* state_in, float* state_out, const void* u_t, const void* delta_t,
                            const float* A, const void* B_t, const void* C_t, const float* Dskip,
                            const void* z_t, const float* delta_bias, int delta_softplus, void* y_t,
                            int64_t batch, int64_t D, int64_t N, ssm_dtype dt, void* stream) {
  return state_update(state_in, state_out, u_t, delta_t, A, B_t, C_t, Dskip, z_t, delta_bias, delta_softplus, y_t,
                      batch, D, N, dt, stream, 0);
}

ssm_status ssm_state_update_zoh(const float* state_in, float* state_out, const void* u_t, const void* delta_t,
                                const float* A, const void* B_t, const void* C_t, const float* Dskip,
                                const void* z_t, const float* delta_bias, int delta_softplus, void* y_t,
                                int64_t batch, int64_t D, int64_t N, ssm_dtype dt, void* stream) {
  return state_update(state_in, state_out, u_t, delta_t, A, B_t, C_t, Dskip, z_t, delta_bias, delta_softplus, y_t,
                      batch, D, N, dt, stream, 1);
}

}  // extern "C"
