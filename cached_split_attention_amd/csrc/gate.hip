// Stand-alone launches of the reuse gates of FlashBlock
// (gist.science/es/paper/2602.05305, section 2, "Estrategias de Reutilizacion
// Adaptativa"); the workgroup bodies (count of changed positions, per-head
// cosine) live in gate_body.h, shared with the attention launch that runs
// the gate in its first workgroups.

#include "gate_body.h"

namespace ba {
namespace {

template <typename W>
__global__ void __launch_bounds__(256) gate_count_kernel(const GateParams p) {
  __shared__ unsigned s_scratch[4];
  gate::count_body<W, false>(p, blockIdx.x, s_scratch);
}

__global__ void __launch_bounds__(256) gate_cos_kernel(const GateParams p) {
  __shared__ double red[3 * 256];
  gate::cos_body(p, blockIdx.x, blockIdx.y, blockIdx.z, red);
}

}  // namespace

int gate_cos_chunks(int n_blk, int d) {
  const int64_t elems = (int64_t)n_blk * d;
  int64_t c = (elems + 8191) / 8192;
  if (c < 1) c = 1;
  if (c > 64) c = 64;
  if (c > n_blk) c = n_blk > 0 ? n_blk : 1;
  return (int)c;
}

size_t gate_workspace_bytes(int mode, int n_seq, int hq, int n_blk, int d) {
  if (mode != BA_GATE_COSINE) return (size_t)n_seq * sizeof(int32_t);
  const size_t nbh = (size_t)n_seq * hq;
  const size_t ints = (nbh * sizeof(int32_t) + 15) & ~(size_t)15;
  return ints + nbh * gate_cos_chunks(n_blk, d) * 3 * sizeof(double);
}

int gate_grid(const GateParams& p) {
  if (p.mode != BA_GATE_COSINE) return (p.n_blk + p.pos_per_wg - 1) / p.pos_per_wg * p.n_seq;
  return p.chunks * p.hq * p.n_seq;
}

hipError_t launch_gate(const GateParams& p, hipStream_t s) {
  if (p.n_seq == 0 || p.n_blk == 0) return hipSuccess;
  if (p.mode != BA_GATE_COSINE) {
    dim3 grid(gate_grid(p));
    if (p.vec16)
      hipLaunchKernelGGL(gate_count_kernel<gate::u32x4>, grid, dim3(256), 0, s, p);
    else if (p.esize == 4)
      hipLaunchKernelGGL(gate_count_kernel<uint32_t>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(gate_count_kernel<uint16_t>, grid, dim3(256), 0, s, p);
  } else {
    dim3 grid(p.chunks, p.hq, p.n_seq);
    hipLaunchKernelGGL(gate_cos_kernel, grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace ba
