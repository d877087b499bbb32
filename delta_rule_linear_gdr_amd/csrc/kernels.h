// Kernel argument blocks and launch entry points of the chunkwise gated
// delta rule (gfx950). Host code in gdr_api.cpp sequences these launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16;

constexpr int CH = 64;    // chunk length
constexpr int DKD = 128;  // key width
constexpr int DVD = 128;  // value width

// Per-chunk intermediates, one tile per (b*H + h, chunk), row-major tiles:
//   W, U, Kt, Qg, R, Rb : 64 x 128 bf16      A, Hm : 64 x 64 bf16
//   h, dh               : 128 x 128 bf16 (key-major: [dk][dv])
//   gn                  : 128 fp32 (exp of the chunk's total log decay)
struct Inter {
    bf16 *W, *U, *Kt, *Qg, *A, *Hm, *h, *R, *dh, *Rb;
    float* gn;
};

struct Shape {
    int64_t B, T, H, NT;
    int vec;   // 1: per-channel gate [B,T,H,128]; 0: scalar gate [B,T,H]
    int f32;   // 1: q,k,v,beta,o,dO,dq,dk,dv,dbeta are fp32; 0: bf16
};

struct Inputs {
    const void *q, *k, *v, *beta, *dO;
    const float *g, *h0, *dht;
};

struct Grads {
    void *dq, *dk, *dv, *dbeta;
    float *dg, *dh0;
};

hipError_t launch_prep(const Shape& s, const Inputs& in, const Inter& it, bool write_A,
                       hipStream_t st);
// Forward state scan: R, h per chunk (when the pointers are set), output o
// (when o != nullptr) and final state ht (when ht != nullptr).
hipError_t launch_scan_fwd(const Shape& s, const Inputs& in, const Inter& it, void* o, float* ht,
                           hipStream_t st);
// Reverse state scan: dh, Rb per chunk and dh0.
hipError_t launch_scan_bwd(const Shape& s, const Inputs& in, const Inter& it, float* dh0,
                           hipStream_t st);
// Chunk-local backward. wy7 selects the expanded seven-product producer.
hipError_t launch_bwd_local(const Shape& s, const Inputs& in, const Inter& it, const Grads& gr,
                            bool wy7, hipStream_t st);

}  // namespace gdr
