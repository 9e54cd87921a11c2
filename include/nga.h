/*
 * nga.h -- C ABI of the neighbour-graph attention library (libnga.so).
 *
 * One step of a neighbour-graph interatomic potential's forward hot path on
 * one MI355X (gfx950) GPU:
 *
 *   nl_build            O(N) cell-list neighbour rows under periodic boundaries
 *   nl_refine           the same rows from cached candidate rows (reuse)
 *   nl_max_displacement the device-side test for that reuse
 *   nl_build_static     nl_build without a workspace, for callers that cannot
 *                       allocate
 *   nl_build_batch      neighbour rows of many structures in one launch sequence
 *   edge_csr            those rows as a destination CSR with image shifts
 *   block_attn_forward  block-dense multi-head attention through the CSR
 *   block_attn_forward_smooth  the same with a per-segment softmax rescale
 *   local_attn_forward  LocalAtten: one query per centre over its edges
 *   block_gather / block_scatter  the padded per-centre block on its own
 *   pair_attn_forward   the same attention by the ragged pair-axis route
 *                       (a measured comparator)
 *   nga_step_graph_*    one step (nl_build, edge_csr, block_attn_forward)
 *                       captured as a HIP graph
 *
 * Sources (web pages, cited by title and section):
 *   [P1] deepmd-kit issue "perf: DPA4 .pt2 LAMMPS (C++ AOTI) inference 3-6x
 *        slower than Python (ASE) due to CPU-side edge construction and data
 *        marshalling".
 *   [P2] deepmd-kit issue "perf: NeighborGraph attention is 4-9x slower than
 *        dense and OOM-prone -- move to block-dense attention via the
 *        destination CSR".
 *   [P4] skill page "ml-mlip-nvalchemi" (batched MLIP inference).
 *
 * Conventions shared by every call:
 *   - Pointers are DEVICE pointers unless their name starts with h_ (host).
 *   - `stream` is a hipStream_t passed as void*.  Every call only enqueues
 *     work on that stream and returns; nothing synchronises except where a
 *     host readback is asked for explicitly (edge_csr's h_n_edges,
 *     nga_sync_status) and in nl_build_batch and the pair-axis comparator,
 *     whose declarations say so.  No call allocates or frees device buffers:
 *     the caller owns every buffer, including the workspace, sized by the
 *     *_workspace_bytes queries (pure host arithmetic); only the step-graph
 *     calls create HIP runtime objects (a stream and a graph).  Keeping the
 *     data on the GPU from positions to outputs, with one optional readback,
 *     is what [P1] "Root cause analysis" and "Proposed optimizations" ask
 *     for.
 *   - Arguments are checked on the host before any HIP call; a bad argument
 *     returns NGA_EINVAL (or NGA_EDTYPE / NGA_EWORKSPACE) and enqueues
 *     nothing.  Errors found by the kernels (a position outside the box, a
 *     row over capacity, too many edges, an index out of range) set bits in
 *     a status word at the start of the workspace; the outputs are then
 *     unspecified, and the error is returned by the next nga_sync_status()
 *     or by edge_csr's readback on that workspace.
 *   - A new workspace must be zero-filled once before its first use (the
 *     status word is cleared only by nga_sync_status / the readback).
 *     Calls that share a workspace must be ordered on one stream.
 *   - HIP runtime failures return NGA_EHIP.
 */
#ifndef NGA_H
#define NGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    NGA_OK = 0,
    NGA_EINVAL = -1,     /* bad argument (host check) */
    NGA_EBOX = -2,       /* a position is not finite or not in [0, L) (device check) */
    NGA_EROWCAP = -3,    /* a centre has more than NGA_ROW_CAP neighbours within rcut */
    NGA_ECAP = -4,       /* the edge count exceeds the caller's capacity */
    NGA_EDTYPE = -5,     /* unsupported dtype */
    NGA_EWORKSPACE = -6, /* workspace missing or smaller than the query returned */
    NGA_EHIP = -7,       /* HIP runtime error */
    NGA_EINDEX = -8,     /* an index in device data is out of range */
    NGA_ETOOBIG = -9     /* more scratch than the allocation-free entry point holds */
};

/* Feature dtypes of the attention calls.
 *   NGA_F64          fp64 features, weights and outputs; fp64 arithmetic.
 *   NGA_F32          fp32 features, weights and outputs; fp32 arithmetic (the
 *                    contractions on the fp32 matrix cores, fp32 accumulation).
 *   NGA_F32_SPLIT16  fp32 features, weights and outputs, softmax and
 *                    accumulation in fp32, but every contraction operand
 *                    carried as two f16 parts (hi + lo, 21-22 significant
 *                    bits after a power-of-two scale) on the f16 matrix
 *                    cores.  Narrower than fp32: asked for by this code only,
 *                    and only for 1, 2 or 4 heads of width 16 with rows up to
 *                    192 (other shapes return NGA_EDTYPE); block_attn_forward
 *                    and block_attn_forward_smooth only. */
enum { NGA_F64 = 0, NGA_F32 = 1, NGA_F32_SPLIT16 = 2 };

/* Neighbours within rcut that nl_build can rank for one centre. */
#define NGA_ROW_CAP 512

/* ------------------------------------------------------------------------ */
/* Neighbour list                                                            */
/* ------------------------------------------------------------------------ */

/* Workspace bytes nl_build needs for n_atoms atoms in the box h_box[3] with
 * cutoff rcut; 0 if the arguments are invalid. */
size_t nl_build_workspace_bytes(int64_t n_atoms, const double* h_box, double rcut);

/*
 * Nearest-sel neighbour rows of every atom under periodic boundaries
 * ([P1] "Root cause analysis": the GPU O(N) cell list of the Python path;
 * [P2] "Measurements": nsel nearest within rcut).
 *
 * pos       [n_atoms][3] fp64, orthorhombic box h_box[3] (x, y, z side
 *           lengths, host), periodic on all axes, every component in [0, L).
 * rcut      cutoff; a neighbour j seen through image n (n in Z^3) is kept if
 *           r2 < rcut*rcut, where d = (x_j - x_i) + n*L per axis and
 *           r2 = (dx*dx + dy*dy) + dz*dz in fp64 without fused multiply-add.
 *           Every image within rcut counts, so boxes smaller than 2*rcut
 *           are allowed (an atom may neighbour itself through n != 0).
 * sel       row width; each row keeps the min(sel, count) smallest keys
 *           (r2, j, n_x, n_y, n_z), ascending, left-packed.
 * nbr       [n_atoms][sel] int32 out: neighbour index j, -1 past the row end.
 * nbr_shift [n_atoms][sel][3] int32 out: image shift n, 0 past the row end.
 * nnei      [n_atoms] int32 out: row length.
 * Limits (else NGA_EINVAL): n_atoms < 2^31; every box side at least rcut/5
 * (image shifts |n| <= 5).  At most NGA_ROW_CAP neighbours within rcut per
 * centre (else NGA_EROWCAP).
 * Device-detected: NGA_EBOX (position outside [0, L) or not finite),
 * NGA_EROWCAP.
 */
int nl_build(const double* pos, int64_t n_atoms, const double* h_box, double rcut, int32_t sel,
             int32_t* nbr, int32_t* nbr_shift, int32_t* nnei, void* ws, size_t ws_bytes,
             void* stream);

/* Device scratch held by nl_build_static, per GPU, for the life of the process. */
#define NGA_STATIC_SCRATCH_BYTES (16u << 20)

/*
 * nl_build for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same rows, bit for bit, with no workspace argument.  Its scratch is a
 * library-held device array of NGA_STATIC_SCRATCH_BYTES per GPU (kept until
 * the process ends); the first call on a GPU looks up that array's address.
 * The call allocates and frees nothing.
 *
 * Arguments as nl_build, except:
 * status    device buffer of at least 256 bytes owned by the caller, zero-
 *           filled once before its first use: device-detected errors
 *           (NGA_EBOX, NGA_EROWCAP) are recorded in it as in a workspace
 *           header, and nga_sync_status(status, stream) returns and clears
 *           them.
 * Limit: nl_build_workspace_bytes(n_atoms, h_box, rcut) must not exceed
 * NGA_STATIC_SCRATCH_BYTES (about 40 bytes per atom plus 12 per cell: some
 * 400,000 atoms at the density of the Fe BCC workloads, 262,000 when the box
 * has the most cells the build uses, two per atom), else NGA_ETOOBIG before
 * anything is enqueued.
 * Every call on one GPU shares that GPU's scratch: calls that can overlap on
 * one GPU (different streams, or threads without ordering) race and must not
 * be issued; calls ordered on one stream are safe.
 */
int nl_build_static(const double* pos, int64_t n_atoms, const double* h_box, double rcut,
                    int32_t sel, int32_t* nbr, int32_t* nbr_shift, int32_t* nnei, void* status,
                    void* stream);

/* Workspace bytes nl_build_batch needs (0 if the structures are invalid). */
size_t nl_build_batch_workspace_bytes(int32_t n_structs, const int64_t* h_atom_ptr,
                                      const double* h_boxes, double rcut);

/*
 * Neighbour rows of a batch of independent periodic structures in one launch
 * sequence ([P4] "Goal": batched inference over many structures at once).
 * Structure b holds atoms h_atom_ptr[b] .. h_atom_ptr[b+1]-1 of pos (all
 * structures' positions concatenated, [N][3], N = h_atom_ptr[n_structs]) in
 * the box h_boxes[3b .. 3b+2].  Its rows name neighbours of the same
 * structure by their index in the concatenated arrays, with image shifts in
 * its own box; the rows of structure b equal nl_build on that structure alone
 * with the indices offset by h_atom_ptr[b].  Outputs as nl_build over N atoms,
 * so edge_csr and the attention calls take the batch as one system.
 * h_atom_ptr [n_structs + 1] (h_atom_ptr[0] = 0, non-decreasing) and h_boxes
 * are host arrays; every structure obeys nl_build's box rules.  The call
 * uploads a small per-structure table into the workspace and synchronises
 * `stream` once (it is not graph-capturable).
 */
int nl_build_batch(const double* pos, int32_t n_structs, const int64_t* h_atom_ptr,
                   const double* h_boxes, double rcut, int32_t sel, int32_t* nbr,
                   int32_t* nbr_shift, int32_t* nnei, void* ws, size_t ws_bytes, void* stream);

/*
 * Neighbour rows of the current positions from candidate rows built earlier
 * by nl_build with a larger cutoff rcut + skin ([P1] "Proposed
 * optimizations": when ago > 0 -- neighbour list unchanged -- reuse what was
 * built instead of rebuilding it).  Each candidate (j, shift) of centre i is
 * re-evaluated with the pinned distance formula at `pos`, those within rcut
 * are kept and ranked by the same total key as nl_build, and the first
 * min(sel, count) are written as rows in nl_build's layout.  The result is
 * bit-identical to nl_build(pos, rcut, sel) as long as the candidate rows
 * hold every pair within rcut: true when no atom has moved more than skin / 2
 * since the candidates were built (see nl_max_displacement) and no candidate
 * row was cut at cand_sel (choose cand_sel above the largest count within
 * rcut + skin).  Positions must move continuously between a candidate build
 * and its refines (not re-wrapped into the box: the stored image shifts
 * assume the candidate-time images).
 *
 * cand_nbr, cand_shift, cand_nnei   nl_build's rows [N][cand_sel] (nnei
 *                                   nullable: rows end at the first -1).
 * cand_sel      <= NGA_ROW_CAP.
 * h_cand_box    the box the candidates were built in; a different h_box
 *               returns NGA_EINVAL (the cached rows belong to another cell).
 * ws            needs only its 256-byte header.
 * Device-detected: NGA_EINDEX (a candidate index or shift out of range).
 */
int nl_refine(const double* pos, int64_t n_atoms, const double* h_box, double rcut, int32_t sel,
              const int32_t* cand_nbr, const int32_t* cand_shift, const int32_t* cand_nnei,
              int32_t cand_sel, const double* h_cand_box, int32_t* nbr, int32_t* nbr_shift,
              int32_t* nnei, void* ws, size_t ws_bytes, void* stream);

/* The largest displacement |pos_i - pos_ref_i| over the atoms, as the plain
 * Euclidean distance (no minimum image), written to the device double *d_max
 * (set to 0 first; enqueued on `stream`, no host synchronisation): the test
 * for reusing candidate rows built at pos_ref, d_max < skin / 2.  An atom
 * re-wrapped into the box since pos_ref therefore reads as a displacement of
 * about one box length and calls for a rebuild (the candidate rows hold image
 * shifts of the pos_ref images).  A non-finite distance reads as +inf.
 * h_box is checked as nl_build checks it; the distance does not use it. */
int nl_max_displacement(const double* pos, const double* pos_ref, int64_t n_atoms,
                        const double* h_box, double* d_max, void* stream);

/* ------------------------------------------------------------------------ */
/* Destination CSR                                                           */
/* ------------------------------------------------------------------------ */

/* Workspace bytes edge_csr needs. */
size_t edge_csr_workspace_bytes(int64_t n_atoms, int32_t sel);

/*
 * Compact padded neighbour rows into the destination CSR
 * ([P1] comments: edge_index, edge_vec, edge_scatter_index, edge_mask built
 * on the device instead of by CPU loops; [P2] "Proposed fix": the
 * destination CSR, destination_row_ptr).
 *
 * nbr, nbr_shift  [n_atoms][sel], [n_atoms][sel][3] int32: nl_build's
 *                 output, or any padded list.  Slot order is kept.
 * nnei            [n_atoms] int32 or NULL.  When given, the first
 *                 min(max(nnei[i], 0), sel) slots of row i are its edges (a
 *                 left-packed list) and must hold indices in [0, n_atoms)
 *                 (else NGA_EINDEX).  When NULL, slot k of row i is an edge
 *                 iff nbr >= 0 (the edge mask).
 * pos, h_box      only read when edge_vec != NULL (fp64 [n_atoms][3], host [3]).
 * row_ptr         [n_atoms+1] int64 out: edges of centre i are
 *                 row_ptr[i] .. row_ptr[i+1]-1 (destination_row_ptr).
 * col             [e_cap] int32 out: source atom j of each edge (edge_index).
 * shift           [e_cap][3] int32 out: image shift n of each edge.
 * dst             [e_cap] int32 out or NULL: centre i of each edge
 *                 (edge_scatter_index).
 * edge_vec        [e_cap][3] fp64 out or NULL: d = (x_j - x_i) + n*L,
 *                 same formula as nl_build.
 * e_cap           edge capacity of the outputs; n_atoms*sel always suffices.
 * h_n_edges       host int64* or NULL.  When given, the call synchronises
 *                 the stream, stores E there, and returns (and clears) any
 *                 device error recorded in this workspace.
 * Device-detected: NGA_ECAP (E > e_cap; only edges below e_cap are written),
 * NGA_EINDEX (an edge's nbr outside [0, n_atoms)).
 */
int edge_csr(const int32_t* nbr, const int32_t* nbr_shift, const int32_t* nnei, int64_t n_atoms,
             int32_t sel, const double* pos, const double* h_box, int64_t* row_ptr,
             int32_t* col, int32_t* shift, int32_t* dst, double* edge_vec, int64_t e_cap,
             int64_t* h_n_edges, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Block-dense neighbour attention                                           */
/* ------------------------------------------------------------------------ */

/* Workspace bytes block_attn_forward needs for these shapes. */
size_t block_attn_workspace_bytes(int dtype, int64_t n_edges, int32_t nnei_cap, int32_t c,
                                  int32_t n_heads, int32_t n_layers);

/*
 * Stacked multi-head self-attention among each centre's edges, gathered
 * through the destination CSR and scattered back to the edge axis
 * ([P2] "Proposed fix: block-dense attention on the graph"; "Graph-native
 * alternatives": per-center self-attention among the center's edges,
 * destination_row_ptr as the segment offsets).
 *
 * For each layer l with weights (Wq, Wk, Wv, Wo) and each centre i with
 * n = row_ptr[i+1] - row_ptr[i] edges e_0 .. e_{n-1}
 * (e_a = order ? order[row_ptr[i] + a] : row_ptr[i] + a):
 *   X = rows x[e_a];  Q = X Wq, K = X Wk, V = X Wv
 *   head h = columns h*d .. h*d+d-1 (d = c / n_heads):
 *     P = softmax over the n keys of (Q_h K_h^T / sqrt(d)), row by row
 *     O_h = P V_h
 *   rows y[e_a] = [O_0 .. O_{H-1}] Wo
 * and the next layer reads y.  Every query attends to every edge of its
 * centre, itself included; there are no biases.
 *
 * dtype      NGA_F64, NGA_F32 or NGA_F32_SPLIT16; x, y and weights are
 *            fp64 for the first, fp32 for the other two.
 * row_ptr    [n_centres+1] int64, row_ptr[0] = 0, non-decreasing.
 * order      [row_ptr[n_centres]] int32 permutation of the edge rows, or
 *            NULL (edges already in destination order, as edge_csr
 *            produces them).
 * n_edges    rows of x and y; row_ptr[n_centres] must not exceed it.
 * nnei_cap   upper bound on any row length (sel); sizes the tiles.
 * weights    [n_layers][4][c][c], matrices q, k, v, o, each row-major
 *            [c_in][c_out] (y = x W).
 * x, y       [n_edges][c]; must not alias.  Rows of y that belong to no
 *            centre are left untouched.
 * Device-detected: NGA_ECAP (row_ptr[n_centres] > n_edges or a row longer
 * than nnei_cap; such rows are skipped), NGA_EINDEX (order out of range).
 */
int block_attn_forward(int dtype, const int64_t* row_ptr, const int32_t* order,
                       int64_t n_centres, int64_t n_edges, int32_t nnei_cap, int32_t c,
                       int32_t n_heads, int32_t n_layers, const void* weights, const void* x,
                       void* y, void* ws, size_t ws_bytes, void* stream);

/*
 * Smooth attention: block_attn_forward with each (query edge, head) segment's
 * softmax rescaled by sum_j e_j / D~, the occupancy-modified weights
 * w_j = softmax_j * (sum_j e_j / D~) of [P2] "Graph-native alternatives"
 * (a per-segment scalar rescale of the vanilla softmax, D~ computed outside
 * the attention).  With e_j = exp(s_j), this is w_j = exp(s_j - ln D~).
 *
 * log_dtilde  [n_layers][n_edges][n_heads] in the dtype of x: ln D~ of the
 *             segment whose query is edge row e (the row of x and y) and
 *             head h, at [l][e][h].  Must not be NULL when n_edges > 0.
 * Other arguments as block_attn_forward.  ln D~ equal to the segment's
 * log-sum-exp gives exactly the vanilla result.  Any finite ln D~ is
 * accepted; as in plain fp32 (fp64) arithmetic, a result beyond the dtype's
 * range comes out as an infinity.
 */
int block_attn_forward_smooth(int dtype, const int64_t* row_ptr, const int32_t* order,
                              int64_t n_centres, int64_t n_edges, int32_t nnei_cap, int32_t c,
                              int32_t n_heads, int32_t n_layers, const void* weights,
                              const void* x, const void* log_dtilde, void* y, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * LocalAtten: attention with the centres as queries and each centre's edges
 * as keys and values, one query per segment ([P2] "Graph-native
 * alternatives": queries = centers, keys = edges, destination_row_ptr as
 * the segment offsets, streamed with the online-softmax recurrence).
 *
 * For each layer l with weights (Wq, Wk, Wv, Wo) and each centre i with
 * edges e_0 .. e_{n-1} (e_a = order ? order[row_ptr[i] + a] : row_ptr[i] + a):
 *   q = xc_i Wq,  k_a = x[e_a] Wk,  v_a = x[e_a] Wv
 *   head h (columns h*d .. h*d+d-1, d = c / n_heads):
 *     w = softmax over a of (q_h . k_a,h / sqrt(d)),  o_h = sum_a w_a v_a,h
 *   yc_i = [o_0 .. o_{H-1}] Wo
 * Stacked layers update the centre rows only (xc <- yc); x is the keys and
 * values of every layer.  A centre without edges gets yc_i = 0.
 *
 * xc, yc      [n_centres][c]; must not alias.
 * x           [n_edges][c] edge features; row_ptr / order as for
 *             block_attn_forward (rows of any length).
 * weights     [n_layers][4][c][c] (q, k, v, o), y = x W.
 * c a multiple of 4 up to 256 and n_heads <= 16 (NGA_EINVAL otherwise).  The
 * workspace holds two [n_centres][n_heads * c] buffers, two [n_heads * c][c]
 * matrices per layer and, for several layers, one [n_centres][c] buffer.
 * Device-detected: NGA_ECAP (row_ptr out of [0, n_edges] or decreasing),
 * NGA_EINDEX (order out of range).
 */
size_t local_attn_workspace_bytes(int dtype, int64_t n_centres, int32_t c, int32_t n_heads,
                                  int32_t n_layers);

int local_attn_forward(int dtype, const int64_t* row_ptr, const int32_t* order,
                       int64_t n_centres, int64_t n_edges, int32_t c, int32_t n_heads,
                       int32_t n_layers, const void* weights, const void* xc, const void* x,
                       void* yc, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* The padded per-centre block, gathered and scattered on its own            */
/* ------------------------------------------------------------------------ */

/*
 * The (nloc, nnei_max, c) block of [P2] "Proposed fix: block-dense attention
 * on the graph", materialised: for every centre i with n_i = row_ptr[i+1] -
 * row_ptr[i] edges (e_k = order ? order[row_ptr[i] + k] : row_ptr[i] + k),
 *   block[i][k][:] = x[e_k][:]   for k < n_i,
 *   block[i][k][:] = 0           for n_i <= k < nnei_cap.
 * block_attn_forward never builds this tensor (its kernels gather straight
 * into on-chip memory); these two calls exist to measure and inspect the
 * gather / scatter boundary on its own.  Both are exact copies.
 *
 * dtype      NGA_F64 or NGA_F32 (element size of x, y and block).
 * row_ptr, order, n_edges as block_attn_forward; n_centres < 2^31.
 * nnei_cap   block rows per centre; a row longer than it is NGA_ECAP.
 * x          [n_edges][c] (gather input); block [n_centres][nnei_cap][c].
 * ws         workspace of at least 256 bytes (its status word), zero-filled
 *            once.
 * Device-detected: NGA_ECAP (row_ptr decreasing, outside [0, n_edges] or a
 * row over nnei_cap: that centre's block is zero-filled / not scattered),
 * NGA_EINDEX (order out of range).
 */
int block_gather(int dtype, const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                 int64_t n_edges, int32_t nnei_cap, int32_t c, const void* x, void* block,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * The inverse: y[e_k][:] = block[i][k][:] for every centre i and k < n_i
 * ([P2] "Proposed fix": scatter back to the edge axis).  Padding rows of the
 * block are not read; rows of y that belong to no centre are left as they
 * are.  Arguments and errors as block_gather; block and y must not alias.
 */
int block_scatter(int dtype, const int64_t* row_ptr, const int32_t* order, int64_t n_centres,
                  int64_t n_edges, int32_t nnei_cap, int32_t c, const void* block, void* y,
                  void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Ragged pair-axis attention (measured comparator)                          */
/* ------------------------------------------------------------------------ */

/* Workspace bytes pair_attn_forward needs for these shapes and chunks of at
 * most pair_chunk pairs; 0 if the arguments are invalid. */
size_t pair_attn_workspace_bytes(int dtype, int64_t n_centres, int64_t n_edges, int32_t c,
                                 int32_t n_heads, int32_t n_layers, int64_t pair_chunk);

/*
 * The same y as block_attn_forward, computed by the ragged pair-axis route
 * that the block-dense path replaces ([P2] "Root cause": enumerate the
 * P = sum_i n_i^2 centre pairs, materialise (P, channels) intermediates, and
 * run segment softmax + index_add over them).  Per layer:
 *   qkv = x [Wq | Wk | Wv] for every edge;
 *   for every pair p = (query edge a, key edge b) of one centre:
 *     prod[p][t] = q_a[t] k_b[t]                      (P x c, materialised)
 *     s[p][h]    = sum over head h's channels of prod[p] / sqrt(d)
 *     m[a][h]    = max over a's pairs of s             (atomic scatter-max)
 *     e[p][h]    = exp(s[p][h] - m[a][h]);  z[a][h] += e[p][h]  (atomic)
 *     w[p][h]    = e[p][h] / z[a][h]
 *     wv[p][t]   = w[p][h(t)] v_b[t]                   (P x c, materialised)
 *     o[a][t]   += wv[p][t]                            (index_add, atomic)
 *   y = o Wo.
 * It exists to be measured beside block_attn_forward; its results agree with
 * it to the floating-point tolerance (atomic accumulation order varies).
 *
 * The pairs are taken in chunks of whole centres holding at most pair_chunk
 * pairs each, so the per-pair tensors need pair_chunk * (c + n_heads)
 * elements plus 8 bytes per pair instead of P * c.
 *
 * Arguments as block_attn_forward, plus pair_chunk >= the largest n_i^2
 * (NGA_EINVAL otherwise) and <= 2^31 - 1.  Unlike the other calls this one
 * synchronises `stream` once, to read row_ptr back and plan the chunks on
 * the host (host memory for n_centres + 1 offsets); everything else is
 * enqueued.  Device-detected: NGA_EINDEX (order out of range).
 */
int pair_attn_forward(int dtype, const int64_t* row_ptr, const int32_t* order,
                      int64_t n_centres, int64_t n_edges, int32_t c, int32_t n_heads,
                      int32_t n_layers, const void* weights, const void* x, void* y,
                      int64_t pair_chunk, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* The step as one HIP graph                                                 */
/* ------------------------------------------------------------------------ */

/*
 * Capture one step -- nl_build, edge_csr without readback, block_attn_forward
 * over x / y of e_cap rows in destination order -- as a HIP graph ([P1]
 * "Proposed optimizations": capture the inference step in a graph to remove
 * the per-kernel launch overhead).  Arguments are those of the three calls;
 * every pointer is baked into the graph, so a replay reads the positions,
 * features and weights those buffers hold at replay time and writes the same
 * outputs; h_box and the other scalars are taken at capture.  Arguments are
 * checked as the calls check them (the error code of the first failing call
 * is returned and no graph is made).  The capture
 * runs on a stream of its own; nothing is launched.  On success *graph_out
 * receives an opaque handle, to be released with nga_step_graph_destroy.
 * Creating a graph allocates host-side and runtime graph objects (no device
 * buffers).  Replays of one graph must be ordered (they share workspaces).
 */
int nga_step_graph_create(const double* pos, int64_t n_atoms, const double* h_box, double rcut,
                          int32_t sel, int32_t* nbr, int32_t* nbr_shift, int32_t* nnei,
                          void* ws_nl, size_t ws_nl_bytes, int64_t* row_ptr, int32_t* col,
                          int32_t* shift, int32_t* dst, double* edge_vec, int64_t e_cap,
                          void* ws_csr, size_t ws_csr_bytes, int dtype, int32_t c,
                          int32_t n_heads, int32_t n_layers, const void* weights, const void* x,
                          void* y, void* ws_attn, size_t ws_attn_bytes, void** graph_out);

/* Launch one replay of a captured step on `stream` (enqueue only). */
int nga_step_graph_launch(void* graph, void* stream);

/* Release a captured step (NULL is accepted). */
int nga_step_graph_destroy(void* graph);

/* ------------------------------------------------------------------------ */
/* Status                                                                    */
/* ------------------------------------------------------------------------ */

/* Synchronise `stream`, then return and clear the first device error
 * recorded in the workspace `ws` (NGA_OK if none). */
int nga_sync_status(void* ws, void* stream);

/* Static description of a status code. */
const char* nga_strerror(int status);

/* Name of the attention kernel block_attn_forward would launch for these
 * shapes, for reporting; never NULL: "fused_f32" (NGA_F32, 1, 2 or 4 heads
 * of 16, rows <= 192), "fused_f32_split16" (NGA_F32_SPLIT16, same shapes),
 * "fused_f64" (fp64, c <= 32, heads of 8 or 16, rows <= 64), "mfma_f64"
 * (fp64, heads of 8, 16 or 32, rows <= 128), "generic_f32", "generic_f64",
 * or "unsupported" for an unknown dtype or a shape NGA_F32_SPLIT16 does not
 * cover. */
const char* nga_attn_variant(int dtype, int32_t nnei_cap, int32_t c, int32_t n_heads);

/* The same, with the layer plan of the fp64 matrix-core path for n_centres
 * centres on the current device, for reporting and tests: "mfma_f64.merged"
 * (per layer a row GEMM for Q, K and V, then one work-group per centre for the
 * attention core and the output projection together: c = 128, heads of 16 or
 * 32, when ceil(n/CUs) rounds of that kernel beat n/CUs rounds of the other
 * plan, 18 ceil(n/CUs) <= 25 n/CUs) or "mfma_f64.per_head" (a row GEMM, the
 * core per (centre, head), a row GEMM for the output projection); both give
 * bit-identical outputs.  Other shapes: nga_attn_variant's name.  Reads the
 * current device's compute-unit count once per device; never NULL.  deepmd-kit
 * issue "perf: NeighborGraph attention is 4-9x slower than dense ...", section
 * "Proposed fix: block-dense attention on the graph". */
const char* nga_attn_plan(int dtype, int64_t n_centres, int32_t nnei_cap, int32_t c,
                          int32_t n_heads);

#ifdef __cplusplus
}
#endif

#endif /* NGA_H */
