// Tile sizes and the launcher table shared by the host layer and the
// per-(dtype, d1, d2) instantiation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace streamkl {

struct FwdArgs;
struct BwdArgs;
struct RaggedTable;
struct DecTable;

constexpr int kFwdRows = 128;     // query rows per forward workgroup (4 waves x 32)
constexpr int kFwdPPRows = 256;   // query rows per ping-pong forward workgroup (8 waves x 32)
constexpr int kFwdTile = 64;      // key rows per forward LDS tile
// key rows per LDS tile of the ping-pong forward: 128 halves its phases
// (each phase has a fixed cost of a barrier and the first LDS reads; 4% faster
// than 64 at 64K); fp32 tiles that large do not fit twice in LDS
template <typename T> constexpr int kFwdPPTile = sizeof(T) == 2 ? 128 : 64;
constexpr int kDecRows = 32;      // longest query range of the decode forward (one wave's rows)
constexpr int kDecBlock = 32;     // key rows per decode-forward block
// waves per dQ workgroup and per separate single-setting dK workgroup: 8
// (two per SIMD) in bf16; 4 in fp32, whose operand fragments would spill at
// two waves per SIMD
template <typename T> constexpr int kBwdWaves = sizeof(T) == 2 ? 8 : 4;
// their query (dQ) or key (dK) rows per workgroup, 32 per wave
constexpr int bwd_rows(bool f32) { return f32 ? 32 * 4 : 32 * 8; }
// key rows per dQ-kernel LDS tile (fp32: 32, whose 64-key tiles spill)
template <typename T> constexpr int kBwdKeyTile = sizeof(T) == 2 ? 64 : 32;
constexpr int kBwdKRows = 128;    // key rows per dK workgroup (4 waves x 32): fused and joint forms
constexpr int kDecBwdTile = 128;  // key rows per tile of the decode backward (4 waves x 32)
// query rows per LDS tile of the dK kernel (fp32 tiles are twice as large)
template <typename T> constexpr int kBwdQTile = sizeof(T) == 2 ? 64 : 32;

// The forward and the single-setting backward launchers take an optional
// ragged-batch table (NULL: a plain launch), as does the decode backward;
// the decode forward takes a table with its split partials' layout.
using FwdLaunch = hipError_t (*)(const FwdArgs&, int64_t, hipStream_t, const RaggedTable*);
using DecFwdLaunch = hipError_t (*)(const FwdArgs&, int64_t, hipStream_t, const DecTable*);
using DqLaunch = hipError_t (*)(const BwdArgs&, int, int64_t, hipStream_t, const RaggedTable*);
using DkLaunch = hipError_t (*)(const BwdArgs&, int, bool, int64_t, hipStream_t, const RaggedTable*);
using DecBwdLaunch = hipError_t (*)(const BwdArgs&, int, int64_t, hipStream_t, const RaggedTable*);

#define SKL_DECL(tn, d1, d2)                                                                                  \
  hipError_t launch_fwd_##tn##_##d1##_##d2(const FwdArgs&, int64_t, hipStream_t, const RaggedTable*);         \
  hipError_t launch_fwd_pp_##tn##_##d1##_##d2(const FwdArgs&, int64_t, hipStream_t, const RaggedTable*);      \
  hipError_t launch_fwd_dec_##tn##_##d1##_##d2(const FwdArgs&, int64_t, hipStream_t, const DecTable*);        \
  hipError_t launch_bwd_dq_##tn##_##d1##_##d2(const BwdArgs&, int, int64_t, hipStream_t, const RaggedTable*); \
  hipError_t launch_bwd_dk_##tn##_##d1##_##d2(const BwdArgs&, int, bool, int64_t, hipStream_t,                \
                                             const RaggedTable*);                                             \
  hipError_t launch_bwd_dec_##tn##_##d1##_##d2(const BwdArgs&, int, int64_t, hipStream_t, const RaggedTable*);
SKL_DECL(f32, 64, 64)
SKL_DECL(f32, 64, 128)
SKL_DECL(f32, 128, 64)
SKL_DECL(f32, 128, 128)
SKL_DECL(bf16, 64, 64)
SKL_DECL(bf16, 64, 128)
SKL_DECL(bf16, 128, 64)
SKL_DECL(bf16, 128, 128)
#undef SKL_DECL

}  // namespace streamkl
