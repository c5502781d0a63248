// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ssm.h"

namespace ssm {

enum class Dt : int { F32 = 0, BF16 = 1 };

struct ScanArgs {
  const void* u;         // [batch][D][L] act
  const void* delta;     // [batch][D][L] act (raw)
  const float* A;        // [D][N]
  const void* Bm;        // [batch][L][N] act
  const void* Cm;        // [batch][L][N] act
  const float* Dskip;    // [D] or null
  const void* z;         // [batch][D][L] act or null
  const float* bias;     // [D] or null
  const float* h0;       // [batch][D][N] initial state or null (zero); may equal final_state
  // fused causal conv1d + SiLU on the input (conv_w null: u is the scan input)
  const float* conv_w = nullptr;  // [D][conv_k]; when set, `u` holds the conv input x
  const float* conv_b = nullptr;  // [D] or null
  int conv_k = 0;                 // 1..4
  void* u_out = nullptr;          // [batch][D][L] act: the conv output (the scan input), or null
  void* y;               // [batch][D][L] act
  float* final_state;    // [batch][D][N] or null
  int64_t batch, L, D;
  int N;
  int softplus;
  int zoh = 0;           // 1: full zero-order hold, input term (exp(Delta A) - 1)/A * B * u
  int ap = 0;            // 1: the arithmetic-progression decay path where a kernel has it
                         //    (SSM_SCAN_AP)
  // [batch][D][ceil(L / kSaveChunk)][N] float32, or null: the state entering each
  // kSaveChunk-token chunk (entry 0 is the initial state), for the backward pass
  // (N <= 16; written by the chunked kernel at 8 tokens per lane, the
  // token-sequential kernel and the sequential kernel)
  float* chunk_states = nullptr;
};

// Tokens per chunk of the saved forward states: the backward pass's chunk at
// N <= 16 (64 lanes x 8 tokens).
constexpr int kSaveChunk = SSM_SAVE_CHUNK;

struct ConvArgs {
  const void* x;       // [batch][D][L] act
  const float* w;      // [D][K]
  const float* bias;   // [D] or null
  void* out;           // [batch][D][L] act
  int64_t batch, D, L;
  int K;               // 1..4
  int silu;            // 0 or 1
};

struct StepArgs {
  const float* state_in;  // [S][D][N]
  float* state_out;       // [S][D][N]
  const void* u;          // [S][D] act
  const void* delta;      // [S][D] act
  const float* A;         // [D][N]
  const void* Bm;         // [S][N] act
  const void* Cm;         // [S][N] act
  const float* Dskip;     // [D] or null
  const void* z;          // [S][D] act or null
  const float* bias;      // [D] or null
  void* y;                // [S][D] act
  int64_t batch, D;
  int N;
  int softplus;
  int zoh = 0;            // 1: full zero-order hold (as ScanArgs::zoh)
};

struct BwdArgs {
  const void* u;          // [batch][D][L] act
  const void* delta;      // [batch][D][L] act (raw)
  const float* A;         // [D][N]
  const void* Bm;         // [batch][L][N] act
  const void* Cm;         // [batch][L][N] act
  const float* Dskip;     // [D] or null
  const void* z;          // [batch][D][L] act or null
  const float* bias;      // [D] or null
  const float* h0;        // [batch][D][N] or null
  const void* dy;         // [batch][D][L] act: gradient of y
  const float* dfinal;    // [batch][D][N] or null: gradient of the final state
  void* du;               // [batch][D][L] act
  void* ddelta;           // [batch][D][L] act (w.r.t. the raw delta)
  float* dA;              // [D][N]
  void* dB;               // [batch][L][N] act
  void* dC;               // [batch][L][N] act
  float* dD;              // [D] or null
  void* dz;               // [batch][D][L] act or null (null whenever z is null)
  float* dbias;           // [D] or null
  float* dh0;             // [batch][D][N] or null
  // [batch][D][ceil(L / kSaveChunk)][N] or null: the forward pass's saved states
  // entering every kSaveChunk-token chunk (entry 0: the initial state)
  const float* chunk_states = nullptr;
  int64_t batch, L, D;
  int N;
  int softplus;
};

struct SsdArgs {
  const void* x;          // [batch][L][H][P] bf16
  const void* dt;         // [batch][L][H] bf16 (raw)
  const float* A;         // [H]
  const void* Bm;         // [batch][L][N] bf16
  const void* Cm;         // [batch][L][N] bf16
  const float* Dskip;     // [H] or null
  const float* dt_bias;   // [H] or null
  const float* h0;        // [batch][H][P][N] or null
  void* y;                // [batch][L][H][P] bf16
  float* final_state;     // [batch][H][P][N] or null
  int64_t batch, L, H;
  int P, N;
  int softplus;
  // set by the launcher: segments per sequence, chunks per segment, the workspace
  int nseg = 1;
  int64_t seg_chunks = 0;
  float* seg_state = nullptr;   // [batch][H][nseg][P][N]
  float* seg_decay = nullptr;   // [batch][H][nseg]
};

// Mamba-2 SSD scan on the matrix cores (P == 64, N in {64, 128}, bfloat16).  A
// workspace of ssd_workspace_bytes lets the sequence run as parallel segments;
// without it (NULL or too small) one segment per sequence.
bool ssd_supported(int64_t H, int64_t P, int64_t N);
size_t ssd_workspace_bytes(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N);
hipError_t launch_ssd_scan(const SsdArgs& a, void* ws, size_t ws_bytes, hipStream_t s);
// The C-ABI SSD call split in two (ssm_api.cpp): argument validation (everything the
// header documents, before any device call; fills *a) and the run on `stream`.
ssm_status ssd_check(const void* x, const void* dt, const float* A, const void* Bm, const void* Cm, const float* Dskip,
                     const float* dt_bias, int dt_softplus, const float* initial_state, const void* y,
                     const float* final_state, int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N,
                     ssm_dtype dtype, const void* workspace, size_t workspace_bytes, SsdArgs* a);
ssm_status ssd_run(const SsdArgs& a, void* workspace, size_t workspace_bytes, void* stream);

// One thread per (b, d) channel, sequential over time.  Any N in [1, 64].
hipError_t launch_scan_sequential(const ScanArgs& a, Dt dt, hipStream_t s);

// Chunked wave-scan kernel.  Returns hipErrorInvalidValue when the shape does not
// fit (callers check chunked_supported first).
bool chunked_supported(const ScanArgs& a, Dt dt, int tokens_per_lane);
// Whether the chunked kernel has a build that saves the chunk states for this shape
// (N == 16 on the vector path); other shapes save through the sequential kernel.
bool chunked_save_supported(const ScanArgs& a);
hipError_t launch_scan_chunked(const ScanArgs& a, Dt dt, int tokens_per_lane, hipStream_t s);

// Token-sequential kernel for many channels: N == 16, L % 8 == 0, 16-byte aligned
// activations, B and C; no fused conv, simplified discretization.  states_per_lane
// 4 (default) or 2.
bool tokseq_supported(const ScanArgs& a);
// Whether the automatic choice runs the token-sequential kernel (measured crossovers).
bool tokseq_preferred(const ScanArgs& a, Dt dt);
hipError_t launch_scan_tokseq(const ScanArgs& a, Dt dt, int states_per_lane, hipStream_t s);

// final_state = initial state, or zeros when src is null (the L == 0 scan).
hipError_t launch_copy_state(float* dst, const float* src, int64_t n, hipStream_t s);

// Backward pass (batch, L, D > 0): float32 workspace of scan_bwd_workspace_bytes
// (saved: the forward pass's chunk states come with the call, BwdArgs::chunk_states).
size_t scan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t D, int N, bool saved);
bool scan_bwd_grid_ok(int64_t batch, int64_t L, int64_t D, int N);
hipError_t launch_scan_bwd(const BwdArgs& a, Dt dt, void* workspace, hipStream_t s);

hipError_t launch_state_update(const StepArgs& a, Dt dt, hipStream_t s);

hipError_t launch_causal_conv1d(const ConvArgs& a, Dt dt, hipStream_t s);

}  // namespace ssm
