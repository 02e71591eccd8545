"""ORACLE — test infrastructure only: the DEER Newton solve, written out.

numpy float64, vectorised over independent channels, sequential over the
steps the pages make sequential.  It follows "Параллельность RNN?"
(forpes.ru), section 1:

* §1.1  residual r(s_{1:T}) = [s_1 - f(s_0), ..., s_T - f(s_{T-1})]; the
  true trajectory is its unique zero.
* §1.2  Newton: solve J(s^(i)) ds = -r(s^(i)), then s^(i+1) = s^(i) + ds;
  J^{-1} is never formed.
* §1.3  J is block-bidiagonal: identity blocks on the diagonal, -df/ds
  evaluated at s_{t-1} on the sub-diagonal, zero elsewhere.
  Level 1: forward substitution ds_1 = -r_1, ds_t = A_t ds_{t-1} - r_t with
  A_t = df/ds(s_{t-1}).
  Level 2: the recurrence is linear, hence associative; closed form
  ds_t = sum_k (A_t ... A_{k+1}) b_k with b = -r, and a pairwise tree over
  log2(T) levels composing the affine maps gives every prefix.

Shapes: states ``s`` are [n, T, S] (S = 1 for ParaGRU, S = 2 (c, h) for
ParaLSTM), initial states ``s0`` [n, S], projections ``u`` [n, T, G], diagonal
weights ``a`` [n, G] (one row per channel).  Jacobians are [n, T, S, S].

Readings of points the pages leave open (each one listed in the design
notes): the Newton start is s^(0) = 0 unless ``s_init`` is given; at
iteration i the residual at s^(i) is evaluated first and the channel stops
if max|r| < tol (``iters`` = updates applied); at the iteration cap the
final residual is evaluated and ``converged`` reports max|r| < tol.
"""
import numpy as np


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


# --------------------------------------------------------------- cells ----

class GRU:
    """ParaGRU: z = sig(a_z h + u_z), r = sig(a_r h + u_r),
    c = tanh(a_c (r h) + u_c), h' = (1 - z) h + z c.  State (h,)."""
    S = 1
    G = 3

    @staticmethod
    def step(s_prev, u, a):
        h = s_prev[..., 0]
        z = _sig(a[..., 0] * h + u[..., 0])
        r = _sig(a[..., 1] * h + u[..., 1])
        c = np.tanh(a[..., 2] * (r * h) + u[..., 2])
        return ((1.0 - z) * h + z * c)[..., None]

    @staticmethod
    def jac(s_prev, u, a):
        """df/dh at (h_{t-1}, u_t), by the chain rule through z, r, c."""
        h = s_prev[..., 0]
        az, ar, ac = a[..., 0], a[..., 1], a[..., 2]
        z = _sig(az * h + u[..., 0])
        r = _sig(ar * h + u[..., 1])
        c = np.tanh(ac * (r * h) + u[..., 2])
        dz = z * (1.0 - z) * az
        dr = r * (1.0 - r) * ar
        dc = (1.0 - c * c) * ac * (r + h * dr)
        return ((1.0 - z) + (c - h) * dz + z * dc)[..., None, None]


class LSTM:
    """ParaLSTM: i, f, o = sig(a h + u), g = tanh(a_g h + u_g),
    c' = f c + i g, h' = o tanh(c').  State (c, h), gate order (i, f, g, o)."""
    S = 2
    G = 4

    @staticmethod
    def _gates(s_prev, u, a):
        h = s_prev[..., 1]
        i = _sig(a[..., 0] * h + u[..., 0])
        f = _sig(a[..., 1] * h + u[..., 1])
        g = np.tanh(a[..., 2] * h + u[..., 2])
        o = _sig(a[..., 3] * h + u[..., 3])
        return i, f, g, o

    @staticmethod
    def step(s_prev, u, a):
        i, f, g, o = LSTM._gates(s_prev, u, a)
        c = f * s_prev[..., 0] + i * g
        return np.stack([c, o * np.tanh(c)], axis=-1)

    @staticmethod
    def jac(s_prev, u, a):
        """2x2 block [[dc'/dc, dc'/dh], [dh'/dc, dh'/dh]] at (s_{t-1}, u_t)."""
        c_prev, h = s_prev[..., 0], s_prev[..., 1]
        ai, af, ag, ao = a[..., 0], a[..., 1], a[..., 2], a[..., 3]
        i, f, g, o = LSTM._gates(s_prev, u, a)
        c = f * c_prev + i * g
        tc = np.tanh(c)
        dc_dc = f
        dc_dh = (c_prev * f * (1.0 - f) * af + g * i * (1.0 - i) * ai
                 + i * (1.0 - g * g) * ag)
        dh_dc = o * (1.0 - tc * tc) * dc_dc
        dh_dh = tc * o * (1.0 - o) * ao + o * (1.0 - tc * tc) * dc_dh
        J = np.empty(c.shape + (2, 2))
        J[..., 0, 0] = dc_dc
        J[..., 0, 1] = dc_dh
        J[..., 1, 0] = dh_dc
        J[..., 1, 1] = dh_dh
        return J


CELLS = {"gru": GRU, "lstm": LSTM}


# ---------------------------------------------------- residual, Jacobian ----

def shifted(s, s0):
    """s_{t-1} for t = 1..T: [s_0, s_1, ..., s_{T-1}]."""
    return np.concatenate([s0[:, None, :], s[:, :-1, :]], axis=1)


def residual(cell, s, s0, u, a):
    """§1.1: r_t = s_t - f(s_{t-1}, u_t), t = 1..T.  [n, T, S]."""
    return s - cell.step(shifted(s, s0), u, a[:, None, :])


def local_jacobians(cell, s, s0, u, a):
    """A_t = df/ds evaluated at (s_{t-1}, u_t), t = 1..T.  [n, T, S, S].
    A_1 multiplies ds_0 = 0 (s_0 is given) and so never acts."""
    return cell.jac(shifted(s, s0), u, a[:, None, :])


def residual_jacobian_dense(cell, s, s0, u, a):
    """§1.3: the full (T*S) x (T*S) Jacobian of r for each channel, built
    block by block — identity on the diagonal, -A_t in block (t, t-1).
    Only for tiny T; [n, T*S, T*S]."""
    n, T, S = s.shape
    A = local_jacobians(cell, s, s0, u, a)
    J = np.zeros((n, T * S, T * S))
    for t in range(T):
        J[:, t * S:(t + 1) * S, t * S:(t + 1) * S] = np.eye(S)
        if t > 0:
            J[:, t * S:(t + 1) * S, (t - 1) * S:t * S] = -A[:, t]
    return J


# -------------------------------------------------------- linear solves ----

def solve_forward_substitution(A, b):
    """§1.3 level 1: ds_1 = b_1, ds_t = A_t ds_{t-1} + b_t (b = -r)."""
    n, T, S = b.shape
    x = np.empty_like(b)
    prev = np.zeros((n, S))
    for t in range(T):
        prev = np.einsum("nij,nj->ni", A[:, t], prev) + b[:, t]
        x[:, t] = prev
    return x


def compose(later, earlier):
    """Affine map composition: apply ``earlier`` = (A1, b1) first, then
    ``later`` = (A2, b2): x -> A2 (A1 x + b1) + b2 = (A2 A1) x + (A2 b1 + b2)."""
    A2, b2 = later
    A1, b1 = earlier
    return (np.einsum("...ij,...jk->...ik", A2, A1),
            np.einsum("...ij,...j->...i", A2, b1) + b2)


def solve_tree_scan(A, b):
    """§1.3 level 2: pairwise tree over ceil(log2 T) levels.  At level k every
    position t >= 2^k composes its running map with the one 2^k steps back
    (all positions of a level in parallel), so after the last level position t
    holds the composition of maps 1..t; applied to ds_0 = 0 this is its b."""
    n, T, S = b.shape
    cur = (A.copy(), b.copy())
    off = 1
    while off < T:
        later = (cur[0][:, off:], cur[1][:, off:])
        earlier = (cur[0][:, :-off], cur[1][:, :-off])
        An, bn = compose(later, earlier)
        nxt = (cur[0].copy(), cur[1].copy())
        nxt[0][:, off:] = An
        nxt[1][:, off:] = bn
        cur = nxt
        off *= 2
    return cur[1]


def solve_closed_form(A, b):
    """§1.3 level 2 closed form, brute force O(T^2):
    ds_t = sum_{k=1..t} (A_t A_{t-1} ... A_{k+1}) b_k."""
    n, T, S = b.shape
    x = np.zeros_like(b)
    for t in range(T):
        acc = np.zeros((n, S))
        for k in range(t + 1):
            P = np.broadcast_to(np.eye(S), (n, S, S)).copy()
            for j in range(t, k, -1):
                P = np.einsum("nij,njk->nik", P, A[:, j])
            acc += np.einsum("nij,nj->ni", P, b[:, k])
        x[:, t] = acc
    return x


def linear_recurrence(A, b, x0=None, reverse=False):
    """The linear recurrence on its own ("Параллельность RNN?", §1.3,
    level 1), step by step: x_t = A_t x_{t-1} + b_t for t = 1..T from x_0, or
    with ``reverse`` x_t = A_t x_{t+1} + b_t for t = T..1 from x_{T+1}
    (``x0`` [n, S] is that boundary value; None means zero)."""
    n, T, S = b.shape
    x = np.empty_like(b)
    prev = np.zeros((n, S)) if x0 is None else np.array(x0, np.float64)
    order = range(T - 1, -1, -1) if reverse else range(T)
    for t in order:
        prev = np.einsum("nij,nj->ni", A[:, t], prev) + b[:, t]
        x[:, t] = prev
    return x


SOLVERS = {
    "serial": solve_forward_substitution,
    "tree": solve_tree_scan,
    "closed": solve_closed_form,
}


# ---------------------------------------------------------------- Newton ----

def newton(cell, u, a, s0, tol, max_iters, s_init=None, solver="serial",
           history=False):
    """DEER Newton solve, per channel.

    Each channel evaluates r at s^(i); it stops if max|r| < tol (NaN counts
    as not converged) or i == max_iters, otherwise applies
    s^(i+1) = s^(i) + ds with ds from the chosen linear solver.

    Returns (s, info) with info = dict(iters [n], converged [n],
    max_abs_res [n], nan [n]) and, if ``history``, info["history"] = list of
    s^(i) for i = 0..max over channels of the updates applied.
    """
    if isinstance(cell, str):
        cell = CELLS[cell]
    n, T, G = u.shape
    S = cell.S
    s = np.zeros((n, T, S)) if s_init is None else np.array(s_init, np.float64)
    active = np.ones(n, bool)
    iters = np.zeros(n, np.int64)
    conv = np.zeros(n, bool)
    mres = np.zeros(n)
    hist = [s.copy()] if history else None
    solve = SOLVERS[solver]
    for it in range(max_iters + 1):
        if not active.any():
            break
        r = residual(cell, s, s0, u, a)
        m = np.abs(r).reshape(n, -1).max(axis=1) if T > 0 else np.zeros(n)
        ok = m < tol  # NaN compares False
        stop = active & (ok | (it == max_iters))
        mres[stop] = m[stop]
        conv[stop] = ok[stop]
        active &= ~stop
        if not active.any():
            break
        idx = np.nonzero(active)[0]
        A = local_jacobians(cell, s[idx], s0[idx], u[idx], a[idx])
        ds = solve(A, -r[idx])
        s[idx] += ds
        iters[idx] += 1
        if history:
            hist.append(s.copy())
    info = dict(iters=iters, converged=conv, max_abs_res=mres,
                nan=np.isnan(mres))
    if history:
        info["history"] = hist
    return s, info


# --------------------------------------------------------------- adjoint ----

def adjoint_dense(cell, s, s0, u, a, g):
    """Adjoint of the converged solve via the transposed §1.3 system:
    J(s*)^T lam = g, with g = dL/ds [n, T, S].  Dense solve, tiny T only.
    Returns lam [n, T, S]."""
    n, T, S = s.shape
    J = residual_jacobian_dense(cell, s, s0, u, a)
    lam = np.linalg.solve(np.transpose(J, (0, 2, 1)), g.reshape(n, T * S)[..., None])
    return lam[..., 0].reshape(n, T, S)


# ------------------------------------------------- layout conversions ----

def from_planes(planes):
    """[B][D][T] planes (one per gate or state component) -> [B*D, T, K]."""
    B, D, T = np.asarray(planes[0]).shape
    return np.stack([np.asarray(p, np.float64).reshape(B * D, T) for p in planes],
                    axis=-1)


def a_per_channel(a, B):
    """[G][D] diagonal weights -> [B*D, G] (channel (b, d) uses a[:, d])."""
    a = np.asarray(a, np.float64)
    return np.tile(a.T, (B, 1))
