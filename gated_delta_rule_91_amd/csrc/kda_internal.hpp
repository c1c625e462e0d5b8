// kda_internal.hpp -- host-side launch entry points of the KDA kernels.
// Each returns hipSuccess or the launch error; arguments were validated by
// the C ABI layer (kda_api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct PrepareArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    char* ws;
    int64_t B, T;            // packed variable-length batches: B = sequences, T = packed tokens
    int64_t row_stride;      // uniform batch: tokens between batch rows of the arrays (0 = T)
    int H, NC;
    float floor_;
    const int32_t* cu_seqlens;   // or null (uniform batch); else [B+1] token offsets
    int64_t* chunk_off;          // with cu_seqlens: [B+1] first chunk of each sequence (written here)
    int32_t* chunk_seq;          // with cu_seqlens: the sequence of each chunk (written here)
};

struct ScanArgs {
    const char* ws;
    const void* g;
    const float* state_in;   // [B,H,dk,dv] or null
    void* out;
    float* state_out;        // [B,H,dk,dv] or null
    float* transition;       // summary mode: [B,H,dk,dk]
    float* zero_state;       // summary mode: [B,H,dk,dv]
    float* states;           // or null; else checkpoints [B,H,ceil(NC/ckpt_every)+1,dk,dv]: slot j is the
                             // state entering chunk j*ckpt_every, the last slot the final state
    int ckpt_every;          // chunks between checkpoints (>= 1 when states is set)
    bool states_tiled;       // with states and ckpt_every 1: the backward's layout (tiled_state_index),
                             // slot NC (the final state) not written
    int64_t B, T;            // packed variable-length batches: B = sequences, T = packed tokens
    int64_t row_stride;      // uniform batch: tokens between batch rows of g and out (0 = T)
    int H, NC;
    const int32_t* cu_seqlens;   // or null (uniform batch); else [B+1] token offsets
    const int64_t* chunk_off;    // with cu_seqlens: [B+1] first chunk of each sequence
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    const void* g;
    float* state;
    void* out;
    int64_t N;
    int H;
    float floor_;
};

struct CombineArgs {
    const float* A;
    const float* Bz;
    const float* s0;
    float* seg_in;
    float* fin;
    int64_t B;
    int n_seg, H, dk, dv;
};

struct BackwardArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* log_alpha;
    const float* beta;
    const void* g;
    const float* state_in;   // [B,H,dk,dv] or null
    const void* d_out;       // [B,T,H,dv] io dtype, or null (zero)
    const float* d_state;    // [B,H,dk,dv] or null (zero)
    void* dq;                // [B,T,H,dk] io dtype
    void* dk;
    void* dv;                // [B,T,H,dv] io dtype
    float* dlog_alpha;       // [B,T,H,dk]
    float* dbeta;            // [B,T,H]
    void* dg;                // [B,T,H,dv] io dtype
    float* d_state_in;       // [B,H,dk,dv] or null
    const void* out;         // the forward output [B,T,H,dv] io dtype (set by launch_backward when it
                             // recomputes the forward)
    char* ws;                // backward_workspace_bytes
    int64_t B, T;            // packed variable-length batches: B = sequences, T = packed tokens
    int H, NC;
    float floor_;
    const int32_t* cu_seqlens;   // or null (uniform batch); else [B+1] token offsets
    const int64_t* chunk_off;    // with cu_seqlens: [B+1] first chunk of each sequence (in the workspace)
    const int32_t* chunk_seq;    // with cu_seqlens: the sequence of each chunk (in the workspace)
};

size_t card_bytes(bool bf16, int dk);
// varlen: a packed batch of B sequences over T tokens (cu_seqlens), whose
// workspace starts with the chunk offsets and chunk -> sequence map
size_t backward_workspace_bytes(bool bf16, int64_t B, int64_t T, int H, int dk, bool varlen = false);
// The forward part of the backward: cards and every chunk's entering state
// into the backward workspace, the output to `out`, the final state to
// state_out (or nowhere).  With a.cu_seqlens set (a packed batch) both calls
// take chunk_off and chunk_seq from the workspace themselves.
hipError_t launch_backward_forward(bool bf16, int dk, const BackwardArgs& a, void* out, float* state_out,
                                   hipStream_t s);
// The backward; recompute: run the forward part first (its output into the
// workspace), else the workspace already holds it and a.out is the output.
hipError_t launch_backward(bool bf16, int dk, const BackwardArgs& a, bool recompute, hipStream_t s);
hipError_t launch_prepare(bool bf16, int dk, const PrepareArgs& a, hipStream_t s);
hipError_t launch_scan(bool bf16, int dk, bool summary, const ScanArgs& a, hipStream_t s);
// segment summaries of bf16 cards at d_k = d_v = 128 with whole 16-column
// slices of [Bz | A] per wave, spw (1 or 2) slices per wave
hipError_t launch_summary_wave(int spw, const ScanArgs& a, hipStream_t s);
hipError_t launch_decode(bool bf16, int dk, const DecodeArgs& a, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

}  // namespace kda
