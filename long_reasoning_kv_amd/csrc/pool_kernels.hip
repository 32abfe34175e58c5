// HIP kernels of the AbridgeKV cache bookkeeping on the device: the append
// of the current token, the device view of a freed block,
// prompt rows, synthetic bulk fills and inspection.
//
// What is computed follows the pages on AbridgeKV (arXiv 2610.20641): the
// abstract and Fig. 1(a) (code rows written by pause tokens, raw block rows
// freed), Fig. 2(a) (the block mask) and Fig. 2(b) (pause token k of block b
// at position P + b*C + bitrev(k)*C/K). RoPE is rotate-half; stored keys are
// rotated in fp64 from the fp64 cos/sin table and rounded once to the pool
// dtype.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../synth/synth_rng.h"
#include "common.h"

namespace abk {

// ---- append the current token (RoPE k at its position, write k and v) ----------

template <typename T, int D>
__global__ void __launch_bounds__(1024) append_kernel(AppendArgs a) {
  const DevPool P = a.P;
  const int i = blockIdx.x;
  const int slot = a.slot[i];
  const int fresh_page = a.new_page[i];
  int32_t* meta = P.meta + (slot * P.L + a.layer) * 4;
  const int n_pers = meta[0], n_open = meta[1], qpos = meta[2];
  const int r = a.compress ? n_open : n_pers;
  int32_t* tab = ptab_of(P, slot, a.layer) + (a.compress ? P.max_pers : 0);
  const int pidx = r / P.pr, srow = r % P.pr;
  const int page = srow == 0 ? fresh_page : tab[pidx];
  const int pos = qpos + 1;
  const T* k = (const T*)a.k + (size_t)i * P.Hkv * D;
  const T* v = (const T*)a.v + (size_t)i * P.Hkv * D;
  T* kd = (T*)P.kpool + ((size_t)page * P.Hkv * P.pr + srow) * D;
  T* vd = (T*)P.vpool + ((size_t)page * P.Hkv * P.pr + srow) * D;
  const double2* rope = P.rope + (size_t)pos * (D / 2);
  for (int t = threadIdx.x; t < P.Hkv * (D / 2); t += blockDim.x) {
    const int hh = t / (D / 2), j = t % (D / 2);
    const T* kr = k + hh * D;
    const double x1 = to_f32(kr[j]), x2 = to_f32(kr[j + D / 2]);
    const double2 cs = rope[j];
    T* kdst = kd + (size_t)hh * P.pr * D;
    kdst[j] = from_f64<T>(rot_first(x1, x2, cs));
    kdst[j + D / 2] = from_f64<T>(rot_second(x1, x2, cs));
    T* vdst = vd + (size_t)hh * P.pr * D;
    vdst[j] = v[hh * D + j];
    vdst[j + D / 2] = v[hh * D + j + D / 2];
  }
  __syncthreads();  // every thread has read meta and the table
  if (threadIdx.x == 0) {
    P.pos[(size_t)page * P.pr + srow] = pos;
    if (srow == 0) tab[pidx] = page;
    meta[a.compress ? 1 : 0] += 1;
    meta[2] = pos;
  }
}

// ---- free: the open block's rows leave the device view ---------------------------

__global__ void free_kernel(FreeArgs a) {
  const int i = blockIdx.x;
  for (int l = threadIdx.x; l < a.P.L; l += blockDim.x)
    a.P.meta[(a.slot[i] * a.P.L + l) * 4 + 1] = 0;
}

// ---- prompt rows -----------------------------------------------------------------

template <typename T, int D>
__global__ void __launch_bounds__(1024) prompt_kernel(PromptArgs a) {
  const DevPool& P = a.P;
  const int r = blockIdx.x;
  if (r == 0 && threadIdx.x == 0) {
    int32_t* meta = P.meta + (a.slot * P.L + a.layer) * 4;
    meta[0] = a.prompt_len;
    meta[1] = 0;
    meta[2] = a.prompt_len - 1;
  }
  if (r == 0) {
    int32_t* tab = ptab_of(P, a.slot, a.layer);
    for (int t = threadIdx.x; t < (a.prompt_len + P.pr - 1) / P.pr; t += blockDim.x)
      tab[t] = a.pages[t];
  }
  if (r >= a.prompt_len) return;
  const int page = a.pages[r / P.pr], srow = r % P.pr;
  const T* k = (const T*)a.k + (size_t)r * a.kv_stride;
  const T* v = (const T*)a.v + (size_t)r * a.kv_stride;
  const double2* rope = P.rope + (size_t)r * (D / 2);
  for (int t = threadIdx.x; t < P.Hkv * (D / 2); t += blockDim.x) {
    const int hh = t / (D / 2), j = t % (D / 2);
    const double x1 = to_f32(k[hh * D + j]), x2 = to_f32(k[hh * D + j + D / 2]);
    const double2 cs = rope[j];
    const size_t o = (((size_t)page * P.Hkv + hh) * P.pr + srow) * D;
    ((T*)P.kpool)[o + j] = from_f64<T>(rot_first(x1, x2, cs));
    ((T*)P.kpool)[o + j + D / 2] = from_f64<T>(rot_second(x1, x2, cs));
    ((T*)P.vpool)[o + j] = v[hh * D + j];
    ((T*)P.vpool)[o + j + D / 2] = v[hh * D + j + D / 2];
  }
  if (threadIdx.x == 0) P.pos[(size_t)page * P.pr + srow] = r;
}

// ---- synthetic fill --------------------------------------------------------------

template <typename T, int D>
__global__ void __launch_bounds__(512) fill_kernel(FillArgs a) {
  const DevPool& P = a.P;
  const int r = blockIdx.x, l = blockIdx.y;
  const int32_t* hdr = a.desc + 4 * l;
  const int pers_off = hdr[0], npers = hdr[1], open_off = hdr[2], nopen = hdr[3];
  const int q = a.quota[l], Kp = a.pause[l];
  const int pers_rows = a.compress ? a.prompt_len + a.nb * q : a.prompt_len + a.G;
  const int open_rows = a.compress ? a.G - a.nb * P.C : 0;
  if (r == 0) {
    int32_t* tab = ptab_of(P, a.slot, l);
    for (int t = threadIdx.x; t < npers; t += blockDim.x) tab[t] = a.desc[pers_off + t];
    for (int t = threadIdx.x; t < nopen; t += blockDim.x) tab[P.max_pers + t] = a.desc[open_off + t];
    if (threadIdx.x == 0) {
      int32_t* meta = P.meta + (a.slot * P.L + l) * 4;
      meta[0] = pers_rows;
      meta[1] = open_rows;
      meta[2] = a.prompt_len + a.G - 1;
    }
  }
  if (r >= pers_rows + open_rows) return;
  int kind, ia, ib, pos, page, srow;
  if (r < a.prompt_len) {
    kind = 0; ia = r; ib = 0; pos = r;
  } else if (r < pers_rows) {
    const int c = r - a.prompt_len;
    if (a.compress) {
      kind = 2; ia = c / q; ib = c % q;
      int nbits = 0;
      while ((1 << nbits) < Kp) ++nbits;
      pos = a.prompt_len + ia * P.C + bitrev_dev(ib, nbits) * (P.C / Kp);
    } else {
      kind = 1; ia = c; ib = 0; pos = r;
    }
  } else {
    kind = 1; ia = a.nb * P.C + (r - pers_rows); ib = 0; pos = a.prompt_len + ia;
  }
  if (r < pers_rows) {
    page = a.desc[pers_off + r / P.pr];
    srow = r % P.pr;
  } else {
    page = a.desc[open_off + (r - pers_rows) / P.pr];
    srow = (r - pers_rows) % P.pr;
  }
  // generate the raw row (stored type) into LDS, then rotate the key; keyed by
  // the model's layer and KV head
  __shared__ float kraw[1024 * 2];  // up to Hkv*D = 1024 elements
  const int n = P.Hkv * D;
  const int ml = l / a.hsplit, mh0 = (l % a.hsplit) * P.Hkv;
  for (int t = threadIdx.x; t < n / 2; t += blockDim.x) {
    const int hh = t / (D / 2), e = t % (D / 2);
    double z0, z1;
    synth_pair(synth_row_key(a.seed, ml, kind, ia, ib, 0, mh0 + hh), e, &z0, &z1);
    kraw[hh * D + 2 * e] = to_f32(from_f32<T>((float)z0));
    kraw[hh * D + 2 * e + 1] = to_f32(from_f32<T>((float)z1));
    synth_pair(synth_row_key(a.seed, ml, kind, ia, ib, 1, mh0 + hh), e, &z0, &z1);
    const size_t o = (((size_t)page * P.Hkv + hh) * P.pr + srow) * D;
    ((T*)P.vpool)[o + 2 * e] = from_f32<T>((float)z0);
    ((T*)P.vpool)[o + 2 * e + 1] = from_f32<T>((float)z1);
  }
  __syncthreads();
  const double2* rope = P.rope + (size_t)pos * (D / 2);
  for (int t = threadIdx.x; t < n / 2; t += blockDim.x) {
    const int hh = t / (D / 2), j = t % (D / 2);
    const double x1 = kraw[hh * D + j], x2 = kraw[hh * D + j + D / 2];
    const double2 cs = rope[j];
    const size_t o = (((size_t)page * P.Hkv + hh) * P.pr + srow) * D;
    ((T*)P.kpool)[o + j] = from_f64<T>(rot_first(x1, x2, cs));
    ((T*)P.kpool)[o + j + D / 2] = from_f64<T>(rot_second(x1, x2, cs));
  }
  if (threadIdx.x == 0) P.pos[(size_t)page * P.pr + srow] = pos;
}

// ---- inspection ------------------------------------------------------------------

template <typename T, int D>
__global__ void read_rows_kernel(ReadArgs a) {
  const DevPool& P = a.P;
  const int rr = blockIdx.x, r = a.row0 + rr;
  const int32_t* meta = meta_of(P, a.slot, a.layer);
  const int32_t* tab = ptab_of(P, a.slot, a.layer);
  const int n_pers = meta[0];
  int page, srow;
  if (r < n_pers) {
    page = tab[r / P.pr];
    srow = r % P.pr;
  } else {
    page = tab[P.max_pers + (r - n_pers) / P.pr];
    srow = (r - n_pers) % P.pr;
  }
  for (int t = threadIdx.x; t < P.Hkv * D; t += blockDim.x) {
    const int hh = t / D, d = t % D;
    const size_t o = (((size_t)page * P.Hkv + hh) * P.pr + srow) * D + d;
    ((T*)a.k_out)[(size_t)rr * P.Hkv * D + t] = ((const T*)P.kpool)[o];
    ((T*)a.v_out)[(size_t)rr * P.Hkv * D + t] = ((const T*)P.vpool)[o];
  }
}

__global__ void export_kernel(ExportArgs a) {
  const DevPool& P = a.P;
  const int32_t* meta = meta_of(P, a.slot, a.layer);
  const int32_t* tab = ptab_of(P, a.slot, a.layer);
  const int n_pers = meta[0], n_open = meta[1];
  const int npp = (n_pers + P.pr - 1) / P.pr, nop = (n_open + P.pr - 1) / P.pr;
  if (threadIdx.x == 0) {
    a.dst[0] = n_pers;
    a.dst[1] = n_open;
    a.dst[2] = meta[2];
    a.dst[3] = npp + nop;
  }
  for (int t = threadIdx.x; t < npp; t += blockDim.x) a.dst[4 + t] = tab[t];
  for (int t = threadIdx.x; t < nop; t += blockDim.x) a.dst[4 + npp + t] = tab[P.max_pers + t];
  int32_t* posd = a.dst + 4 + npp + nop;
  for (int r = threadIdx.x; r < n_pers + n_open; r += blockDim.x) {
    int page, srow;
    if (r < n_pers) {
      page = tab[r / P.pr];
      srow = r % P.pr;
    } else {
      page = tab[P.max_pers + (r - n_pers) / P.pr];
      srow = (r - n_pers) % P.pr;
    }
    posd[r] = P.pos[(size_t)page * P.pr + srow];
  }
}

// ---- launchers ---------------------------------------------------------------------

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const int th = threads_for(a.P.Hkv, a.P.D);
  ABK_DISPATCH_TD(a.P.dtype, a.P.D,
                  hipLaunchKernelGGL((append_kernel<T, DD>), dim3(a.n), dim3(th), 0, s, a));
  return hipGetLastError();
}

hipError_t launch_free(const FreeArgs& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(free_kernel, dim3(a.n), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prompt(const PromptArgs& a, hipStream_t s) {
  const int th = threads_for(a.P.Hkv, a.P.D);
  const int rows = a.prompt_len > 0 ? a.prompt_len : 1;
  ABK_DISPATCH_TD(a.P.dtype, a.P.D,
                  hipLaunchKernelGGL((prompt_kernel<T, DD>), dim3(rows), dim3(th), 0, s, a));
  return hipGetLastError();
}

hipError_t launch_fill(const FillArgs& a, int32_t max_rows, hipStream_t s) {
  const int rows = max_rows > 0 ? max_rows : 1;
  ABK_DISPATCH_TD(a.P.dtype, a.P.D,
                  hipLaunchKernelGGL((fill_kernel<T, DD>), dim3(rows, a.P.L), dim3(512), 0, s, a));
  return hipGetLastError();
}

hipError_t launch_read(const ReadArgs& a, hipStream_t s) {
  if (a.nrows == 0) return hipSuccess;
  ABK_DISPATCH_TD(a.P.dtype, a.P.D,
                  hipLaunchKernelGGL((read_rows_kernel<T, DD>), dim3(a.nrows), dim3(256), 0, s, a));
  return hipGetLastError();
}

hipError_t launch_export(const ExportArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(export_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}
}  // namespace abk
